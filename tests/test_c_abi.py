"""include/mk.h is a C interface: a plain C99 program that includes it
compiles with every warning an error, links against the library, and runs
the host-only entry points (version, error strings, the plan check, the unit
listing, the address model, argument checks of the GPU entry points) with no
GPU and no Python in between; and every structure it declares has the
layout (size, each field's offset and size) the binding's ctypes mirror
assumes."""
import ctypes as C
import os
import shutil
import subprocess

import pytest

from persistent_interpreter_amd import binding as B, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mk.h"

static mk_config tiny(void) {
  mk_config c;
  memset(&c, 0, sizeof c);
  c.n_layers = 2; c.hidden = 256; c.n_q_heads = 4; c.n_kv_heads = 2; c.head_dim = 64;
  c.ffn_dim = 688; c.vocab = 1024; c.rms_eps = 1e-5f; c.rope_theta = 10000.0f;
  c.tied_embeddings = 1; c.qk_norm = 0; c.max_batch = 1; c.max_seq = 48;
  return c;
}

int main(void) {
  mk_config c = tiny();
  mk_plan_report rep;
  mk_addr_report arep;
  mk_unit_info units[4096];
  int32_t q_off[17];
  int32_t pos = 16, tok = 5;
  mk_handle *h = (mk_handle *)0;
  int n, i, pages = 0;
  printf("version %d\n", mk_version());
  printf("strerror %s\n", mk_strerror(MK_ERR_UNSUPPORTED));
  if (mk_plan_check(&c, 1, 16, 20, 0, 7u, &rep) != MK_OK) { printf("plan %s\n", rep.msg); return 1; }
  printf("plan instr %d groups %d pages %d sim %d/%d\n", rep.n_instr, rep.n_groups, rep.n_pages,
         rep.sim_errors, rep.sim_runs);
  n = mk_plan_units(&c, 1, 16, units, 4096, q_off);
  if (n != rep.n_instr || q_off[16] != n) return 2;
  for (i = 0; i < n; ++i) pages += units[i].pages;
  if (pages != rep.n_pages) return 3;
  if (mk_addr_check(&c, 1, 16, 4, &pos, &tok, 0, &arep) != MK_OK) { printf("addr %s\n", arep.msg); return 4; }
  if (mk_addr_check_launch(&c, 1, 16, 4, &pos, &tok, 0, &arep) != MK_OK) return 5;
  printf("addr accesses %lld\n", (long long)arep.accesses);
  c.head_dim = 96;
  if (mk_plan_check(&c, 1, 16, 0, 0, 0u, &rep) != MK_ERR_UNSUPPORTED) return 6;
  /* the GPU entry points check their arguments before touching a device */
  if (mk_create((const mk_config *)0, (const mk_weights *)0, &h) != MK_ERR_INVALID_ARG || h) return 7;
  if (mk_decode_step(h, 1, &tok, &pos, (void *)0, (float *)0, (void *)0) != MK_ERR_INVALID_ARG) return 8;
  if (mk_sync_status(h) != MK_ERR_INVALID_ARG) return 9;
  mk_destroy(h);
  printf("ok\n");
  return 0;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(B.LIB_PATH):
        build.build()
    src = tmp_path / "use_mk.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_mk"
    lib_dir = os.path.dirname(os.path.abspath(B.LIB_PATH))
    libname = os.path.basename(B.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        os.path.join(lib_dir, libname), f"-Wl,-rpath,{lib_dir}"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    run = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=300)
    assert run.returncode == 0, run.stdout
    out = run.stdout
    assert f"version {B.lib().mk_version()}" in out and out.rstrip().endswith("ok")
    assert "sim 0/20" in out


STRUCTS = {"mk_config": B.MkConfig, "mk_layer_weights": B.MkLayerWeights, "mk_weights": B.MkWeights,
           "mk_plan_report": B.MkPlanReport, "mk_unit_info": B.MkUnitInfo,
           "mk_addr_report": B.MkAddrReport}


def test_struct_layouts_match_the_binding(tmp_path):
    """Every structure the header declares has, field by field, the offset
    and the size the ctypes mirror in the binding gives it."""
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "mk.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname}.{f} %zu %zu\\n", offsetof({cname}, {f}), '
                         f'sizeof((({cname} *)0)->{f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-o", str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    got = {}
    for line in subprocess.run([str(exe)], stdout=subprocess.PIPE, text=True, check=True).stdout.splitlines():
        key, *vals = line.split()
        got[key] = tuple(int(v) for v in vals if v.isdigit())
    for cname, py in STRUCTS.items():
        assert got[cname] == (C.sizeof(py),), cname
        for f, _ in py._fields_:
            d = getattr(py, f)
            assert got[f"{cname}.{f}"] == (d.offset, d.size), (cname, f)


def test_readme_c_example_compiles(tmp_path):
    """The C usage example of the README compiles against the header as
    strict C99 and links against the library."""
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    import re
    text = open(os.path.join(ROOT, "README.md")).read()
    m = re.search(r"<!-- c-example -->\s*```c\n(.*?)```\s*<!-- /c-example -->", text, flags=re.S)
    assert m, "the README has no C example"
    src = tmp_path / "example.c"
    src.write_text(m.group(1) + "\nint main(void) { return 0; }\n")
    lib_dir = os.path.dirname(os.path.abspath(B.LIB_PATH))
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                        os.path.join(ROOT, "include"), str(src), "-o", str(tmp_path / "example"),
                        B.LIB_PATH, f"-Wl,-rpath,{lib_dir}"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
