"""Several greedy decode steps in one launch (mk_decode_steps_greedy).

Bar: bitwise equality with the same steps run as chained one-step launches
(mk_decode_step_greedy) from the same start: the logits of every step, the
final tokens and positions, and the whole KV cache.  The one-step path is
held to the oracle by the parity tests; splitting the steps over launches
changes no arithmetic (same schedule, same reduction order), only where the
step boundary is, so any difference is a protocol error: a stale token, a
K/V row read before an earlier step of the launch wrote it, a counter
target off by a step.  Runs under MK_FLAG_PERTURB (seeded random delays
before every instruction of every wave) widen the interleavings."""
import numpy as np
import pytest
import torch

from persistent_interpreter_amd import binding as B, harness, synth

pytestmark = pytest.mark.gpu

# name, batch, launch sizes (their sum is the step count), kv_splits,
# workgroups (0: one per CU), flags of the multi-step handle
CASES = [
    ("tiny", 1, (5, 1, 6), 0, 0, 0),
    ("tiny", 1, (12,), 1, 0, 0),                    # one split: paged K/V
    ("tiny", 1, (4, 8), 0, 3, B.MK_FLAG_PERTURB),   # 3 workgroups, delays
    ("tiny_qk", 1, (3, 5), 0, 0, 0),                # head_dim 128, q/k norm
    ("tiny", 3, (4, 4), 0, 0, 0),
    ("tiny", 3, (2, 6), 1, 3, B.MK_FLAG_PERTURB),
    ("tiny", 8, (8,), 0, 2, 0),
    ("llama1b", 1, (16,), 0, 0, 0),
    pytest.param("llama1b_b8", 8, (8,), 0, 0, 0, marks=pytest.mark.timeout(600)),
]


def _start(mc, batch):
    kv = synth.make_kv_cache(mc, filled=mc.prior) if batch == 1 else synth.make_kv_cache(mc)
    return kv, synth.make_tokens(mc, batch), synth.make_positions(mc, batch)


@pytest.mark.parametrize("name,batch,launches,splits,cus,flags", CASES)
def test_launch_of_n_steps_equals_n_launches(name, batch, launches, splits, cus, flags):
    steps = sum(launches)
    mc = synth.CONFIGS[name]
    if batch > 1 and mc.batch != batch:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    mc = mc.replace(steps=steps)
    W = synth.make_weights(mc, threads=16)
    dW = harness.upload_weights(W)
    kv, tok, pos = _start(mc, batch)
    print(f"case: {name} batch {batch} launches {launches} splits {splits} "
          f"workgroups {cus or 'all'} flags {flags}", flush=True)
    a = harness.Session(mc, dW, kv.copy(), batch=batch, kv_splits=splits, num_cus=cus)
    a.set_inputs(tok, pos)
    ref = []
    for i in range(steps):
        assert a.step_greedy() == B.MK_OK
        ref.append(a.logits.clone())
    assert a.mk.sync_status() == B.MK_OK

    b = harness.Session(mc, dW, kv.copy(), batch=batch, kv_splits=splits, num_cus=cus,
                        flags=flags)
    b.set_inputs(tok, pos)
    done = 0
    for n in launches:
        lg = torch.full((n, batch, mc.vocab), float("nan"), dtype=torch.float32, device="cuda")
        rc = b.mk.decode_steps_greedy(batch, n, b.tokens, b.positions, b.kv, lg,
                                      b.tokens, b.positions)
        assert rc == B.MK_OK, rc
        assert b.mk.sync_status() == B.MK_OK
        for s in range(n):
            if not torch.equal(lg[s].view(torch.int32), ref[done + s].view(torch.int32)):
                d = float((lg[s] - ref[done + s]).abs().max())
                pytest.fail(f"{name}: logits of step {done + s} (launch step {s} of {n}) "
                            f"differ, max |d| {d:.3e}")
        done += n
        assert torch.equal(b.positions.cpu(), torch.as_tensor(pos + done, dtype=torch.int32))
    assert torch.equal(b.tokens, a.tokens)
    assert torch.equal(b.positions, a.positions)
    assert torch.equal(b.kv, a.kv)
    a.close()
    b.close()


def test_separate_outputs_leave_inputs_alone():
    """With next_tokens / next_positions apart from the inputs, the inputs
    stay as given, the tokens are the last step's and the positions advance
    by the step count; a later one-step greedy call continues the chain
    (the greedy counters account for every step of the launch)."""
    mc = synth.CONFIGS["tiny"].replace(steps=10)
    W = synth.make_weights(mc)
    dW = harness.upload_weights(W)
    kv, tok, pos = _start(mc, 1)
    a = harness.Session(mc, dW, kv.copy())
    a.set_inputs(tok, pos)
    ref = []
    for i in range(7):
        assert a.step_greedy() == B.MK_OK
        ref.append(a.logits.clone())
    b = harness.Session(mc, dW, kv.copy())
    b.set_inputs(tok, pos)
    nt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    npos = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros(6, 1, mc.vocab, dtype=torch.float32, device="cuda")
    print("case: tiny, 6 steps in one launch, separate outputs", flush=True)
    assert b.mk.decode_steps_greedy(1, 6, b.tokens, b.positions, b.kv, lg, nt, npos) == B.MK_OK
    assert b.mk.sync_status() == B.MK_OK
    assert int(b.tokens.cpu()[0]) == int(tok[0])
    assert int(b.positions.cpu()[0]) == int(pos[0])
    assert int(npos.cpu()[0]) == int(pos[0]) + 6
    for s in range(6):
        assert torch.equal(lg[s].view(torch.int32), ref[s].view(torch.int32)), s
    assert int(nt.cpu()[0]) == int(torch.argmax(lg[5, 0]))
    # one more greedy step through the one-step entry point
    b.tokens.copy_(nt)
    b.positions.copy_(npos)
    assert b.step_greedy() == B.MK_OK
    assert b.mk.sync_status() == B.MK_OK
    assert torch.equal(b.logits.view(torch.int32), ref[6].view(torch.int32))
    a.close()
    b.close()


def test_position_past_capacity_ends_the_launch():
    """A launch whose later steps would pass max_seq: the kernel's own input
    check reports a bad position at that step (every wave exits), the steps
    before it are complete, and the handle recovers."""
    mc = synth.CONFIGS["tiny"].replace(steps=4)
    W = synth.make_weights(mc)
    dW = harness.upload_weights(W)
    kv, tok, pos = _start(mc, 1)
    max_seq = kv.shape[4]
    a = harness.Session(mc, dW, kv.copy())
    start = max_seq - 2
    a.set_inputs(tok, np.array([start], np.int32))
    ref = []
    for i in range(2):
        assert a.step_greedy() == B.MK_OK
        ref.append(a.logits.clone())
    assert a.mk.sync_status() == B.MK_OK
    b = harness.Session(mc, dW, kv.copy())
    b.set_inputs(tok, np.array([start], np.int32))
    lg = torch.zeros(4, 1, mc.vocab, dtype=torch.float32, device="cuda")
    print(f"case: tiny, 4 steps from position {start} of {max_seq}", flush=True)
    assert b.mk.decode_steps_greedy(1, 4, b.tokens, b.positions, b.kv, lg,
                                    b.tokens, b.positions) == B.MK_OK
    assert b.mk.sync_status() == B.MK_ERR_BAD_POSITION
    for s in range(2):
        assert torch.equal(lg[s].view(torch.int32), ref[s].view(torch.int32)), s
    # recovered: a valid launch runs
    b.set_inputs(tok, pos)
    assert b.mk.decode_steps_greedy(1, 2, b.tokens, b.positions, b.kv, lg,
                                    b.tokens, b.positions) == B.MK_OK
    assert b.mk.sync_status() == B.MK_OK
    a.close()
    b.close()
