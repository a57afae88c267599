"""Random shapes through the host entry points (tests/host_fuzz.py): plain
library in this process, and the host-sanitized build (AddressSanitizer +
UBSan over the scheduler, plan checker and address model) in a child
process with the sanitizer runtimes preloaded."""
import os
import subprocess
import sys

import pytest

import host_fuzz
from persistent_interpreter_amd import binding as B, build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("seed", [1, 2])
def test_random_shapes_plan_and_stay_in_bounds(seed):
    res = host_fuzz.run(seed, 60)
    assert res[B.MK_OK] >= 30 and res[B.MK_ERR_INVALID_ARG] > 0


def test_random_shapes_under_host_sanitizers(tmp_path):
    pre = build.sanitizer_preload()
    if pre is None:
        pytest.skip("g++ has no ASan/UBSan runtime here")
    lib = build.build_sanitized(str(tmp_path / "libmk_san.so"))
    env = dict(os.environ, MK_LIB_PATH=lib, LD_PRELOAD=pre,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_fuzz.py"), "3", "30"], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    assert r.returncode == 0 and "clean" in r.stdout, r.stdout[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
