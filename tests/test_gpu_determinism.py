"""Determinism and failure handling of the persistent kernel on the GPU.

An ordering bug in a persistent kernel does not fail loudly: it shows as a
rare wrong token after many steps ("Quand ne pas le faire", section 9.3).
Every reduction here runs in an order fixed by the schedule (no float
atomics), so two handles stepping the same inputs must give bitwise equal
logits at every step, also when one of them runs under MK_FLAG_PERTURB
(seeded random delays before every instruction of every wave), and a wait
that can never complete must end in the watchdog with every wave exiting.

Each run stops at its first mismatching step and names it."""
import numpy as np
import pytest
import torch

import oracle as O
from persistent_interpreter_amd import binding as B, harness, synth

pytestmark = pytest.mark.gpu


def _lockstep(mc, steps, batch=1, flags_b=0, **knobs):
    """Two handles from the same start, device-chained greedy steps; the
    logits compared bitwise after every step."""
    W = synth.make_weights(mc, threads=16)
    kv = synth.make_kv_cache(mc, filled=mc.prior) if batch == 1 else synth.make_kv_cache(mc)
    tok, pos = synth.make_tokens(mc, batch), synth.make_positions(mc, batch)
    dW = harness.upload_weights(W)
    a = harness.Session(mc, dW, kv.copy(), batch=batch, **knobs)
    b = harness.Session(mc, dW, kv.copy(), batch=batch, flags=flags_b, **knobs)
    for s in (a, b):
        s.set_inputs(tok, pos)
    for i in range(steps):
        assert a.step_greedy() == B.MK_OK and b.step_greedy() == B.MK_OK
        if not torch.equal(a.logits.view(torch.int32), b.logits.view(torch.int32)):
            d = float((a.logits - b.logits).abs().max())
            pytest.fail(f"{mc.name}: logits differ at step {i} (max |d| {d:.3e})")
        if not torch.equal(a.tokens, b.tokens):
            pytest.fail(f"{mc.name}: greedy tokens differ at step {i}")
    assert a.mk.sync_status() == B.MK_OK and b.mk.sync_status() == B.MK_OK
    assert torch.equal(a.kv, b.kv)
    a.close()
    b.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("start,splits", [(512, 0), (0, 64)], ids=["paged", "registers"])
def test_llama1b_1000_steps_bitwise(start, splits):
    """1000 chained greedy steps of the Llama-1B shape: from 512 prior
    positions (long splits: paged attention), and from an empty cache with
    64 splits of at most 16 positions (the register-path attention the
    512-position bench runs)."""
    steps = 1000
    mc = synth.CONFIGS["llama1b"].replace(prior=start, steps=steps)
    print(f"case: llama1b from position {start}, kv_splits {splits}, {steps} steps", flush=True)
    _lockstep(mc, steps, kv_splits=splits)


@pytest.mark.timeout(600)
def test_llama1b_batch8_200_steps_bitwise():
    mc = synth.CONFIGS["llama1b_b8"].replace(steps=200)
    print("case: llama1b batch 8, 200 steps", flush=True)
    _lockstep(mc, 200, batch=8)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,batch,splits", [("tiny", 1, 0), ("tiny", 1, 1), ("tiny", 8, 0),
                                               ("llama1b", 1, 0)])
def test_perturbed_interleavings_give_the_same_bits(name, batch, splits):
    """One handle runs with seeded random delays before every instruction of
    every wave: other interleavings of the same schedule, same bits."""
    mc = synth.CONFIGS[name]
    if batch > 1:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    steps = 32 if name == "tiny" else 16
    print(f"case: {name} batch {batch} splits {splits} perturbed, {steps} steps", flush=True)
    _lockstep(mc, steps, batch=batch, flags_b=B.MK_FLAG_PERTURB, kv_splits=splits)


def test_unsatisfiable_wait_ends_in_the_watchdog():
    """The host raises one counter target by one, so the LM units' wait can
    never complete: the step ends through the kernel's own watchdog
    (20 ms here), mk_sync_status reports MK_ERR_DEVICE_TIMEOUT, and the
    device runs a following step of another handle correctly."""
    mc = synth.CONFIGS["tiny"]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    print("case: tiny, forced unsatisfiable wait", flush=True)
    s = harness.Session(mc, W, kv.copy(), flags=B.MK_FLAG_TEST_STALL, watchdog_ms=20)
    s.set_inputs(tok, pos)
    assert s.step() == B.MK_OK                       # enqueued
    assert s.mk.sync_status() == B.MK_ERR_DEVICE_TIMEOUT
    s.close()
    print("case: tiny, a valid step after the watchdog", flush=True)
    ok = harness.Session(mc, W, kv.copy())
    ok.set_inputs(tok, pos)
    ok.step_checked()
    lg = ok.logits.cpu().numpy()
    ok.close()
    ref = O.decode_step(mc, O.upcast_weights(W), tok, pos, kv.copy())
    assert float(np.abs(lg - ref).max()) <= 2e-2
    assert int(np.argmax(lg[0])) == int(np.argmax(ref[0]))
