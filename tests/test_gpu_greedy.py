"""The greedy next token chosen inside the launch (mk_decode_step_greedy).

Bars: the token equals the first arg max of the fp32 logits the same launch
wrote (an integer: exact), the position advances by one, and steps chained on
the device (the kernel overwrites its own token and position inputs) feed
exactly the tokens that host-side greedy decoding feeds."""
import numpy as np
import pytest
import torch

import oracle as O
from persistent_interpreter_amd import binding as B
from persistent_interpreter_amd import harness, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,steps", [("tiny", 32), ("llama1b", 32)])
def test_device_chain_matches_host_greedy(name, steps):
    mc = synth.CONFIGS[name]
    W = synth.make_weights(mc, threads=16)
    dW = harness.upload_weights(W)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    print(f"case: {name} host greedy, {steps} steps", flush=True)
    a = harness.Session(mc, dW, kv.copy())
    fed_h, out_h = harness.greedy_run(a, tok, pos, steps)
    a.close()
    print(f"case: {name} device-chained greedy, {steps} steps", flush=True)
    s = harness.Session(mc, dW, kv.copy())
    s.set_inputs(tok, pos)
    for i in range(steps):
        fed = s.tokens.cpu().numpy().copy()
        assert np.array_equal(fed, fed_h[i]), (i, fed, fed_h[i])
        assert int(s.positions.cpu()[0]) == int(pos[0]) + i
        rc = s.step_greedy()
        assert rc == B.MK_OK, rc
        assert s.mk.sync_status() == B.MK_OK
        lg = s.logits.cpu().numpy()
        # the kernel is deterministic: same schedule, same reduction order
        assert np.array_equal(lg, out_h[i]), i
        assert int(s.tokens.cpu()[0]) == int(np.argmax(lg[0])), i
    assert int(s.positions.cpu()[0]) == int(pos[0]) + steps
    s.close()


def test_separate_outputs_leave_inputs_alone():
    mc = synth.CONFIGS["tiny"]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    s = harness.Session(mc, W, kv)
    s.set_inputs(tok, pos)
    nt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    npos = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    print("case: tiny greedy step with separate outputs", flush=True)
    rc = s.mk.decode_step_greedy(1, s.tokens, s.positions, s.kv, s.logits, nt, npos)
    assert rc == B.MK_OK
    assert s.mk.sync_status() == B.MK_OK
    assert int(s.tokens.cpu()[0]) == int(tok[0])
    assert int(s.positions.cpu()[0]) == int(pos[0])
    lg = s.logits.cpu().numpy()
    assert int(nt.cpu()[0]) == int(np.argmax(lg[0]))
    assert int(npos.cpu()[0]) == int(pos[0]) + 1
    # a plain step in between, then a greedy one: the greedy arrival count
    # must not depend on plain steps
    assert s.step() == B.MK_OK
    rc = s.mk.decode_step_greedy(1, s.tokens, s.positions, s.kv, s.logits, nt, npos)
    assert rc == B.MK_OK
    assert s.mk.sync_status() == B.MK_OK
    assert int(nt.cpu()[0]) == int(np.argmax(s.logits.cpu().numpy()[0]))
    s.close()


def test_exact_tie_goes_to_the_lower_index():
    """With O and down projections zero, h_L is the embedding row of the fed
    token t, so (tied head, unit norm weights) logit_v = E_v . x with x the
    RMS-normed E_t.  E_t is scaled by 4 (exact in bf16) and copied into a
    lower row; by Cauchy-Schwarz the two identical rows hold the largest
    logit, equal on both sides, and the lower index must win."""
    mc = synth.CONFIGS["tiny"]
    W = synth.make_weights(mc)
    for lw in W["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    t, low = 700, 5
    row = O.f32_to_bf16(O.bf16_to_f32(W["embed"][t]) * np.float32(4.0))
    assert np.array_equal(O.bf16_to_f32(row), O.bf16_to_f32(W["embed"][t]) * 4)
    W["embed"] = W["embed"].copy()
    W["embed"][t] = row
    W["embed"][low] = row
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    pos = synth.make_positions(mc)
    tok = np.array([t], np.int32)
    ref = O.decode_step(mc, W, tok, pos, kv.copy())
    assert ref[0, low] == ref[0, t] and int(np.argmax(ref[0])) == low
    s = harness.Session(mc, W, kv)
    s.set_inputs(tok, pos)
    print("case: tiny greedy tie", flush=True)
    assert s.step_greedy() == B.MK_OK
    assert s.mk.sync_status() == B.MK_OK
    lg = s.logits.cpu().numpy()[0]
    assert lg[low] == lg[t], (lg[low], lg[t])
    assert lg[t] == lg.max()
    assert int(s.tokens.cpu()[0]) == low
    assert int(s.positions.cpu()[0]) == int(pos[0]) + 1
    s.close()


def test_cooperative_launch_gives_the_same_steps():
    """MK_FLAG_COOPERATIVE only changes how the grid is launched."""
    mc = synth.CONFIGS["tiny"]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    runs = []
    for flags in (0, B.MK_FLAG_COOPERATIVE):
        print(f"case: tiny 4 greedy steps, flags {flags}", flush=True)
        s = harness.Session(mc, W, kv.copy(), flags=flags)
        runs.append(harness.greedy_run(s, tok, pos, 4))
        s.close()
    for a, b in zip(runs[0][1], runs[1][1]):
        assert np.array_equal(a, b)
