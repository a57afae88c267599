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


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link the library; returns its path.
    ``defines`` (e.g. ``["MK_SDEPTH=2"]``) override compile-time knobs."""
    out_dir = os.path.dirname(out)
    os.makedirs(out_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    objs = []
    stem = os.path.splitext(os.path.basename(out))[0]
    for src in ("mk_kernel.hip", "mk_probe.hip"):
        o = os.path.join(out_dir, f"{stem}_" + src.replace(".hip", ".o"))
        _run([HIPCC, *DEVICE_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", o])
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


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
