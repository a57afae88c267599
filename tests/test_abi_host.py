"""Host-only tests of the C-ABI library: it loads, exports every entry
point include/mk.h declares, validates arguments without a GPU, and its
scheduler's plans pass the static checks and simulated interleavings (and a
deliberately broken plan is caught).  No compute call needs a GPU here."""
import ctypes as C
import os
import re

import pytest

from persistent_interpreter_amd import binding as B
from persistent_interpreter_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(B.LIB_PATH):
        from persistent_interpreter_amd import build
        build.build()
    return B.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"mk_create", "mk_decode_step", "mk_destroy"} <= set(names)
    lib = C.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_version_and_strerror():
    assert B.lib().mk_version() == 109
    for code in (0, -1, -2, -3, -4, -5, -6, -10, -11, -12, -99):
        assert len(B.strerror(code)) > 0


def test_null_arguments_rejected_without_gpu():
    L = B.lib()
    out = C.c_void_p()
    assert L.mk_create(None, None, C.byref(out)) == B.MK_ERR_INVALID_ARG
    cfg = B.make_config(synth.CONFIGS["tiny"])
    assert L.mk_create(C.byref(cfg), None, C.byref(out)) == B.MK_ERR_INVALID_ARG
    assert L.mk_create(C.byref(cfg), None, None) == B.MK_ERR_INVALID_ARG
    assert L.mk_decode_step(None, 1, None, None, None, None, None) == B.MK_ERR_INVALID_ARG
    assert L.mk_decode_step_greedy(None, 1, None, None, None, None, None, None,
                                   None) == B.MK_ERR_INVALID_ARG
    assert L.mk_decode_steps_greedy(None, 1, 4, None, None, None, None, None, None,
                                    None) == B.MK_ERR_INVALID_ARG
    assert L.mk_sync_status(None) == B.MK_ERR_INVALID_ARG
    assert L.mk_stream_read(None, 16, None, None) == B.MK_ERR_INVALID_ARG
    L.mk_destroy(None)  # NULL-safe


@pytest.mark.parametrize("field,value,code", [
    ("n_kv_heads", 3, B.MK_ERR_UNSUPPORTED),     # 4 % 3 != 0
    ("head_dim", 96, B.MK_ERR_UNSUPPORTED),
    ("hidden", 260, B.MK_ERR_UNSUPPORTED),       # not a multiple of 8
    ("kv_splits", 65, B.MK_ERR_UNSUPPORTED),
    ("n_layers", 0, B.MK_ERR_INVALID_ARG),
    ("max_seq", 0, B.MK_ERR_INVALID_ARG),
    ("n_layers", 4097, B.MK_ERR_UNSUPPORTED),    # layer index is 16-bit
    ("hidden", (1 << 20) + 8, B.MK_ERR_UNSUPPORTED),   # K pieces per row are 16-bit
    ("ffn_dim", (1 << 20) + 8, B.MK_ERR_UNSUPPORTED),
])
def test_bad_configs(field, value, code):
    cfg = B.make_config(synth.CONFIGS["tiny"])
    setattr(cfg, field, value)
    rc, rep = B.plan_check(cfg, 1, 8)
    assert rc == code, rep.msg


def test_attention_width_limit():
    """The O projection's contraction (n_q_heads * head_dim) has the same
    16-bit piece count as hidden and ffn_dim."""
    cfg = B.make_config(synth.CONFIGS["tiny"])
    cfg.n_kv_heads, cfg.n_q_heads = 8192, 16384      # 16384 x 64 = 2^20: the limit
    assert b"2^20" not in B.plan_check(cfg, 1, 8)[1].msg
    cfg.n_kv_heads, cfg.n_q_heads = 8200, 16400
    rc, rep = B.plan_check(cfg, 1, 8)
    assert rc == B.MK_ERR_UNSUPPORTED and b"2^20" in rep.msg


def test_batch_out_of_range():
    cfg = B.make_config(synth.CONFIGS["tiny"], max_batch=2)
    assert B.plan_check(cfg, 3, 8)[0] == B.MK_ERR_INVALID_ARG
    assert B.plan_check(cfg, 0, 8)[0] == B.MK_ERR_INVALID_ARG


def test_batch_above_eight_unsupported():
    """Positions and per-sequence 1/rms of a step are staged in LDS for at
    most 8 sequences."""
    cfg = B.make_config(synth.CONFIGS["tiny"], max_batch=16)
    assert B.plan_check(cfg, 8, 8)[0] == B.MK_OK
    assert B.plan_check(cfg, 9, 8)[0] == B.MK_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,cus,batch", [
    ("tiny", 256, 1), ("tiny", 13, 1), ("tiny", 1, 1), ("tiny", 8, 3), ("tiny", 256, 8),
    ("llama1b", 256, 1), ("llama1b", 31, 1), ("llama1b", 256, 8), ("llama1b", 256, 3),
    ("llama1b", 13, 7), ("tiny", 13, 5),
    ("qwen3_8b", 256, 1), ("llama70b", 256, 4)])
def test_plans_validate(name, cus, batch):
    mc = synth.CONFIGS[name]
    cfg = B.make_config(mc, max_batch=max(batch, 1))
    runs = 4 if mc.n_layers > 2 else 40
    rc, rep = B.plan_check(cfg, batch, cus, sim_runs=runs, seed=7)
    assert rc == B.MK_OK, rep.msg
    assert rep.sim_errors == 0 and rep.sim_runs == runs
    # every weight byte of the model is streamed exactly once per step
    norms = (2 * mc.n_layers + 1) * mc.hidden * 2
    if mc.qk_norm:
        norms += 2 * mc.n_layers * mc.head_dim * 2
    expect = mc.weight_bytes() - norms
    assert rep.weight_bytes == expect
    assert rep.max_cu_bytes * cus >= rep.weight_bytes


def test_adversarial_interleavings_7160():
    """The count of adversarial schedules validated by the static
    schedule-synthesis work cited on the megakernel index page."""
    cfg = B.make_config(synth.CONFIGS["tiny"])
    rc, rep = B.plan_check(cfg, 1, 16, sim_runs=7160, seed=2026)
    assert rc == B.MK_OK, rep.msg
    assert rep.sim_runs == 7160 and rep.sim_errors == 0


@pytest.mark.parametrize("corrupt", [1, 2, 3])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_corrupted_plans_are_caught(corrupt, seed):
    cfg = B.make_config(synth.CONFIGS["tiny"])
    rc, rep = B.plan_check(cfg, 1, 16, sim_runs=200, corrupt=corrupt, seed=seed)
    assert rc != B.MK_OK
    assert rep.sim_errors > 0 and rep.msg


@pytest.mark.parametrize("corrupt", [1, 2, 3])
@pytest.mark.parametrize("name,batch", [("tiny", 1), ("tiny", 3), ("llama1b", 1)])
def test_plan_errors_in_one_workgroup_are_caught(name, batch, corrupt):
    """On one workgroup every producer is in the consumer's own queue, which
    the interleavings run in order; the static happens-before check must
    still find the dropped signal, the short target or the dropped wait (the
    kernel's roles pipeline, so queue order orders nothing in memory)."""
    mc = synth.CONFIGS[name]
    cfg = B.make_config(mc, max_batch=batch)
    assert B.plan_check(cfg, batch, 1)[0] == B.MK_OK
    rc, rep = B.plan_check(cfg, batch, 1, sim_runs=0, corrupt=corrupt, seed=3)
    assert rc != B.MK_OK and b"no wait orders" in rep.msg, rep.msg


@pytest.mark.parametrize("name,batch,cus", [("tiny", 1, 256), ("tiny", 3, 3), ("llama1b", 1, 256),
                                           ("llama1b_b8", 8, 256)])
def test_two_writers_of_the_same_rows_are_caught(name, batch, cus):
    """One O unit's rows grown into the next O unit's: every activation
    element must have exactly one writer (a split-K down group counts as one,
    its last arrival writing the rows)."""
    mc = synth.CONFIGS[name]
    cfg = B.make_config(mc, max_batch=batch)
    assert B.plan_check(cfg, batch, cus)[0] == B.MK_OK
    rc, rep = B.plan_check(cfg, batch, cus, corrupt=5)
    assert rc != B.MK_OK and b"write the same elements" in rep.msg, rep.msg


@pytest.mark.parametrize("name", ["tiny", "llama1b", "tiny_qk", "llama70b"])
def test_out_of_range_split_is_caught(name):
    """The extent check: an attention unit whose split index is one past
    the last would address partials and K/V rows outside their buffers."""
    cfg = B.make_config(synth.CONFIGS[name], max_batch=1)
    rc, rep = B.plan_check(cfg, 1, 256, corrupt=4)
    assert rc != B.MK_OK
    assert b"out of range" in rep.msg


@pytest.mark.parametrize("name,over", [("tiny_qk", dict(head_dim=64)),      # q/k norm needs hd 128
                                       ("tiny", dict(n_q_heads=6, n_kv_heads=2)),  # 3 q heads per KV head
                                       ("tiny", dict(head_dim=96))])
def test_unsupported_shapes_refused_before_the_device(name, over):
    """Shapes the kernels cannot run are refused by mk_create after the
    argument checks and before any device call: q/k norm only with head_dim
    128 (the paged attention body norms and rotates pairs (d, d + 64)),
    query heads per KV head dividing the 8 compute waves, head_dim 64 or
    128."""
    mc = synth.CONFIGS[name].replace(**over)
    cfg = B.make_config(mc, max_batch=1, max_seq=64)
    dummy = C.c_void_p(0x1000)  # never dereferenced on this path
    layers = (B.MkLayerWeights * mc.n_layers)()
    for ly in layers:
        for f, _ in B.MkLayerWeights._fields_:
            setattr(ly, f, dummy)
    w = B.MkWeights(dummy, dummy, dummy, layers)
    out = C.c_void_p()
    assert B.lib().mk_create(C.byref(cfg), C.byref(w), C.byref(out)) == B.MK_ERR_UNSUPPORTED
    assert not out.value


@pytest.mark.parametrize("name,batch,paged,splits", [("llama1b", 1, 0, 0), ("qwen3_8b", 1, 1, 0),
                                                    ("llama1b_b8", 8, 1, 4), ("tiny", 3, 0, 3)])
def test_plan_report_kernel_choice(name, batch, paged, splits):
    """The report names the attention body (paged K/V or register prefetch)
    and the split-K down projection of batched plans (one split per MLP
    chunk: 4 for Llama-1B, 3 for the tiny shape whose FFN has 3 pieces)."""
    mc = synth.CONFIGS[name]
    cfg = B.make_config(mc, max_batch=batch)
    rc, rep = B.plan_check(cfg, batch, 256)
    assert rc == B.MK_OK, rep.msg
    assert rep.paged_kv == paged and rep.down_splits == splits


@pytest.mark.parametrize("name", ["tiny_qk", "qwen3_8b", "llama70b"])
def test_head_dim_128_shapes_plan(name):
    """The q/k-norm and head_dim-128 shapes plan and validate (their
    attention runs on paged K/V)."""
    cfg = B.make_config(synth.CONFIGS[name], max_batch=1)
    rc, rep = B.plan_check(cfg, 1, 256, sim_runs=2)
    assert rc == B.MK_OK, rep.msg


def _declared_params():
    """name -> parameter declarations, from include/mk.h."""
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(mk_[a-z_]+)\s*\(([^;{]*?)\)\s*;", src, flags=re.S):
        params = m.group(2).strip()
        out[m.group(1)] = [] if params in ("", "void") else [" ".join(p.split()) for p in params.split(",")]
    return out


_SCALARS = {"int32_t": (4, True), "int": (4, True), "uint32_t": (4, False),
            "uint64_t": (8, False), "size_t": (8, False)}


def test_binding_signatures_match_the_header():
    """Every entry point is called through a ctypes prototype that matches
    the header argument by argument: pointers as pointers, integers with the
    declared width and signedness (a missing or short prototype would pass a
    64-bit pointer as a 32-bit int)."""
    L = B.lib()
    decl = _declared_params()
    assert set(decl) == set(B.EXPORTED)
    for name, params in decl.items():
        f = getattr(L, name)
        assert f.argtypes is not None and len(f.argtypes) == len(params), name
        for p, t in zip(params, f.argtypes):
            if "*" in p:
                assert t is C.c_void_p or issubclass(t, C._Pointer), (name, p, t)
            else:
                size, signed = _SCALARS[p.split()[0]]
                assert C.sizeof(t) == size, (name, p, t)
                assert (t(-1).value < 0) == signed, (name, p, t)


def test_plan_units_count_only_and_partial_fill():
    """mk_plan_units: with no array it returns the count; with a short array
    it fills that many entries, leaves the rest alone and still returns the
    full count; bad arguments are refused."""
    L = B.lib()
    cfg = B.make_config(synth.CONFIGS["tiny"])
    n = L.mk_plan_units(C.byref(cfg), 1, 16, None, 0, None)
    assert n > 0
    units = (B.MkUnitInfo * 8)()
    for u in units:
        u.op = -7
    assert L.mk_plan_units(C.byref(cfg), 1, 16, units, 5, None) == n
    assert all(units[i].op in range(1, 8) for i in range(5))
    assert all(units[i].op == -7 for i in range(5, 8))
    assert L.mk_plan_units(C.byref(cfg), 1, 16, None, 5, None) == B.MK_ERR_INVALID_ARG
    assert L.mk_plan_units(C.byref(cfg), 0, 16, None, 0, None) == B.MK_ERR_INVALID_ARG
    assert L.mk_plan_units(None, 1, 16, None, 0, None) == B.MK_ERR_INVALID_ARG
