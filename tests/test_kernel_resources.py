"""Register, scratch and LDS budget of the persistent kernels, from the
compiler's resource report of the in-tree build (written by
persistent_interpreter_amd.build as _lib/libmk_resources.json).

A workgroup is 12 waves of 64 lanes on one CU of 4 SIMDs, so every
instantiation must fit 3 waves per SIMD (at most 168 VGPRs + AGPRs per
lane), and its LDS is all dynamic (the 160 KB the launch asks for).  The
register-path one-step kernels, which run the Llama-1B batch-1 and batch-8
steps at one step per launch, keep every value in registers: a spill there
sits on a critical path (four spills in the RMSNorm piece loop once cost
about 10 us a step).  The paged and multi-step instantiations do spill; the
bound below only catches a large regression."""
import json
import os

import pytest

from persistent_interpreter_amd import build

RES = os.path.join(build.OUT_DIR, "libmk_resources.json")
KERNELS = [f"{k}<{p}>" for k in ("mk_interp", "mk_interp_n", "mk_interp_b", "mk_interp_bn")
           for p in ("false", "true")]


@pytest.fixture(scope="module")
def res():
    if not os.path.exists(RES):
        build.build()
    with open(RES) as f:
        return json.load(f)


def test_every_instantiation_is_reported(res):
    assert set(KERNELS) <= set(res)


@pytest.mark.parametrize("k", KERNELS)
def test_one_workgroup_of_12_waves_fits_a_cu(res, k):
    r = res[k]
    assert r["Occupancy [waves/SIMD]"] >= 3
    assert r["VGPRs"] + r["AGPRs"] <= 168
    assert r["LDS Size [bytes/block]"] == 0          # dynamic LDS only
    assert r["ScratchSize [bytes/lane]"] <= 256
    assert r["Dynamic Stack"] in ("False", 0, False)


@pytest.mark.parametrize("k", ["mk_interp<false>", "mk_interp_b<false>"])
def test_register_path_one_step_kernels_do_not_spill(res, k):
    assert res[k]["VGPRs Spill"] == 0 and res[k]["ScratchSize [bytes/lane]"] == 0


def test_report_parser_on_a_remark_sample():
    text = "\n".join([
        "x.hip:1:1: remark: Function Name: _ZN2mk9mk_interpILb1EEEvPKNS_6DevCtxE [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs: 168 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs Spill: 28 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:2:1: remark: Function Name: _ZN2mk12mk_fill_zeroEPjj [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:2:1: remark:     VGPRs: 4 [-Rpass-analysis=kernel-resource-usage]",
    ])
    got = build.parse_resource_usage(text)
    assert got == {"mk_interp<true>": {"VGPRs": 168, "VGPRs Spill": 28, "Dynamic Stack": "False"},
                   "mk_fill_zero": {"VGPRs": 4}}
