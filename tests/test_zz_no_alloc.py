"""mk_decode_step_static (the entry point that allocates nothing) against
mk_decode_step_greedy on the same inputs, through the C ABI.

Both run the same kernel on the same schedule; only where the step's scratch
lives differs (the library's static per-GPU array, cleared by a fill kernel
on every call, instead of the plan's own buffers), so the logits, the written
K/V cache, the next tokens and positions must be bitwise identical.  Two
calls in a row, the second with a smaller input (batch 3 on the batched
kernel, then batch 1), show that the array's leftover contents from one call
do not reach the next."""
import numpy as np
import pytest
import torch

from persistent_interpreter_amd import binding as B, harness, synth

pytestmark = pytest.mark.gpu


def _case(batch, steps=3):
    mc = synth.CONFIGS["tiny"]
    if batch > 1:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    return mc, W, kv, tok, pos


def _compare(sess_ref, sess_st, batch, tok, pos, steps):
    """`steps` chained greedy steps on each session from the same start."""
    for s in (sess_ref, sess_st):
        s.set_inputs(tok, pos)
    for i in range(steps):
        assert sess_ref.step_greedy() == B.MK_OK
        rc = sess_st.mk.decode_step_static(batch, sess_st.tokens, sess_st.positions, sess_st.kv,
                                           sess_st.logits, sess_st.tokens, sess_st.positions)
        assert rc == B.MK_OK, B.strerror(rc)
        assert sess_ref.mk.sync_status() == B.MK_OK and sess_st.mk.sync_status() == B.MK_OK
        a, b = sess_ref.logits.cpu().numpy(), sess_st.logits.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (batch, i, float(np.abs(a - b).max()))
        assert torch.equal(sess_ref.tokens, sess_st.tokens) and torch.equal(sess_ref.positions, sess_st.positions)
    assert np.array_equal(sess_ref.kv_host(), sess_st.kv_host())


def test_static_scratch_matches_the_allocating_step():
    # a larger call (batch 3, batched kernel), then a smaller one (batch 1)
    for batch in (3, 1):
        mc, W, kv, tok, pos = _case(batch)
        print(f"case: tiny batch {batch}, positions {pos.tolist()}", flush=True)
        ref = harness.Session(mc, W, kv.copy(), batch=batch)
        st = harness.Session(mc, W, kv.copy(), batch=batch)
        # no schedule for this batch size on `st` yet: refused, nothing launched
        rc = st.mk.decode_step_static(batch, st.tokens, st.positions, st.kv, st.logits,
                                      st.tokens, st.positions)
        assert rc == B.MK_ERR_NOT_PREPARED
        # one ordinary step builds the schedule (on a scratch copy of the cache)
        scratch_kv = st.kv.clone()
        st.set_inputs(tok, pos)
        assert st.mk.decode_step(batch, st.tokens, st.positions, scratch_kv, st.logits) == B.MK_OK
        assert st.mk.sync_status() == B.MK_OK
        _compare(ref, st, batch, tok, pos, steps=3)
        ref.close()
        st.close()


def test_a_schedule_beyond_the_array_is_refused():
    """450 layers of the tiny shape need more than 32 MiB of counters."""
    mc = synth.CONFIGS["tiny"].replace(n_layers=450)
    W = synth.make_weights(mc, threads=16)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    s = harness.Session(mc, W, kv.copy())
    s.set_inputs(tok, pos)
    s.step_checked()  # builds the schedule (allocating step)
    rc = s.mk.decode_step_static(1, s.tokens, s.positions, s.kv, s.logits, None, None)
    assert rc == B.MK_ERR_UNSUPPORTED
    s.close()
