"""Build the C-ABI library ``_lib/libmk.so`` in-tree for gfx950.

Device code is compiled with hipcc for gfx950 only; the host-side scheduler
and ABI are plain C++ (g++) against the HIP runtime headers.  Packed fp32
instructions are disabled for all device code.

    python -m persistent_interpreter_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libmk.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include", "-Wall", "-Wno-unused-function"]
# host-only checking build: the C++ scheduler, plan checker and address
# model under AddressSanitizer and UBSan (g++ only; device code is untouched)
SAN_LIB = os.path.join(OUT_DIR, "libmk_san.so")
SAN_HOST_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
                  "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def parse_resource_usage(text: str) -> dict:
    """The compiler's per-kernel resource remarks (VGPRs, AGPRs, SGPRs,
    spills, scratch bytes per lane, occupancy in waves per SIMD, static LDS)
    as {kernel: {field: int}}, kernels named as in the source
    (``mk_interp<false>`` ...)."""
    import re
    res, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: (.*?) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        t = m.group(1).strip()
        if t.startswith("Function Name:"):
            mangled = t.split(":", 1)[1].strip()
            k = re.match(r"_ZN2mk(\d+)(\w+)", mangled)
            name = k.group(2)[:int(k.group(1))] if k else mangled
            tpl = re.match(r"_ZN2mk\d+\w+?ILb([01])EE", mangled)
            if tpl:
                name += "<true>" if tpl.group(1) == "1" else "<false>"
            cur = res.setdefault(name, {})
        elif cur is not None and ":" in t:
            key, val = t.split(":", 1)
            try:
                cur[key.strip()] = int(val.strip())
            except ValueError:
                cur[key.strip()] = val.strip()
    return res


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link the library; returns its path.
    ``defines`` (e.g. ``["MK_SDEPTH=2"]``) override compile-time knobs.
    The kernels' resource usage goes to ``<stem>_resources.json`` beside it."""
    out_dir = os.path.dirname(out)
    os.makedirs(out_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    objs = []
    stem = os.path.splitext(os.path.basename(out))[0]
    for src in ("mk_kernel.hip", "mk_probe.hip"):
        o = os.path.join(out_dir, f"{stem}_" + src.replace(".hip", ".o"))
        remarks = ["-Rpass-analysis=kernel-resource-usage"] if src == "mk_kernel.hip" else []
        text = _run([HIPCC, *DEVICE_FLAGS, *remarks, *dflags, "-c", os.path.join(CSRC, src), "-o", o])
        if remarks:
            import json
            with open(os.path.join(out_dir, f"{stem}_resources.json"), "w") as f:
                json.dump(parse_resource_usage(text), f, indent=1, sort_keys=True)
        objs.append(o)
    for src in ("mk_sched.cpp", "mk_abi.cpp", "mk_addr.cpp"):
        o = os.path.join(out_dir, f"{stem}_" + src.replace(".cpp", ".o"))
        _run(["g++", *HOST_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64"])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_sanitized(out: str = SAN_LIB) -> str:
    """The library with its host code under AddressSanitizer and UBSan, for
    CPU-only checks of the host entry points (mk_plan_check, mk_plan_units,
    mk_addr_check*).  The device objects are the plain build's (built first
    if missing).  A process that loads it needs the sanitizer runtimes
    preloaded (``sanitizer_preload()``)."""
    kobj = os.path.join(OUT_DIR, "libmk_mk_kernel.o")
    pobj = os.path.join(OUT_DIR, "libmk_mk_probe.o")
    if not (os.path.exists(kobj) and os.path.exists(pobj)):
        build()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    stem = os.path.splitext(os.path.basename(out))[0]
    objs = [kobj, pobj]
    for src in ("mk_sched.cpp", "mk_abi.cpp", "mk_addr.cpp"):
        o = os.path.join(os.path.dirname(out), f"{stem}_" + src.replace(".cpp", ".o"))
        _run(["g++", *HOST_FLAGS, *SAN_HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    tmp = out + ".tmp"
    _run(["g++", "-shared", *SAN_HOST_FLAGS, *objs, "-o", tmp, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, out)
    return out


def sanitizer_preload() -> Optional[str]:
    """LD_PRELOAD value with g++'s ASan and UBSan runtimes, or None if the
    toolchain has none."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        r = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
        path = r.stdout.strip()
        if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
            return None
        libs.append(path)
    return " ".join(libs)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
