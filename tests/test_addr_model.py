"""Host address model of the decode kernel (mk_addr_check): every global
access of every role, per lane, for every unit and step of a plan lies in the
buffer it addresses.  This gates each kernel path before it runs on a GPU.

The model's own sensitivity is pinned by planting size errors: a buffer one
record short must be reported at the access site that reaches that record."""
import pytest

from persistent_interpreter_amd import binding as B, synth

CUS = 256


def _check(name, steps, batch=None, corrupt=0, **over):
    mc = synth.CONFIGS[name]
    if over:
        mc = mc.replace(**over)
    batch = batch or mc.batch
    cfg = B.make_config(mc, max_batch=batch)
    pos = synth.make_positions(mc, batch)
    tok = synth.make_tokens(mc, batch)
    return B.addr_check(cfg, batch, CUS, steps, pos, tok, corrupt)


@pytest.mark.parametrize("name,steps", [("tiny", 32), ("tiny_qk", 32), ("llama1b", 2),
                                        ("qwen3_8b", 1)])
def test_every_access_in_bounds(name, steps):
    """All steps of a greedy run (positions p .. p+steps-1, the last one the
    cache's final slot for the tiny shapes)."""
    rc, rep = _check(name, steps)
    assert rep.accesses > 0
    assert rc == 0 and rep.violations == 0, rep.msg.decode()


def test_last_slot_and_position_zero():
    """The first and the last cache slot (an empty cache; a full one)."""
    mc = synth.CONFIGS["tiny_qk"]
    cfg = B.make_config(mc)
    for p in (0, mc.max_seq - 1):
        rc, rep = B.addr_check(cfg, 1, CUS, 1, [p], [mc.vocab - 1])
        assert rc == 0, (p, rep.msg.decode())


def test_fewer_workgroups_and_splits():
    """Other schedules of the same shape: 8 workgroups, 1 and 5 KV splits."""
    mc = synth.CONFIGS["tiny_qk"]
    for cus, splits in ((8, 0), (CUS, 1), (CUS, 5)):
        cfg = B.make_config(mc, kv_splits=splits)
        rc, rep = B.addr_check(cfg, 1, cus, 4, synth.make_positions(mc),
                               synth.make_tokens(mc))
        assert rc == 0, (cus, splits, rep.msg.decode())


@pytest.mark.parametrize("name", ["tiny", "tiny_qk"])
@pytest.mark.parametrize("corrupt,site", [(1, "kv_cache"), (2, "partials"), (3, "rope"),
                                          (4, "q"), (5, "h")])
def test_planted_size_errors_are_found(name, corrupt, site):
    rc, rep = _check(name, 32, corrupt=corrupt)
    msg = rep.msg.decode()
    assert rc != 0 and rep.violations > 0
    assert f"at {site}+" in msg, msg


@pytest.mark.parametrize("batch,cus", [(3, 3), (8, 2), (8, 256)])
def test_wide_lm_units_in_bounds(batch, cus):
    """Batched LM-head units of up to 512 rows (tiny shape on 2 and 3
    workgroups, Llama-1B shape on 256)."""
    name = "tiny" if cus < 256 else "llama1b_b8"
    mc = synth.CONFIGS[name].replace(batch=batch, pos_lo=4, pos_hi=40)
    cfg = B.make_config(mc, max_batch=batch)
    rc, rep = B.addr_check(cfg, batch, cus, 2, synth.make_positions(mc, batch), synth.make_tokens(mc, batch))
    assert rc == 0 and rep.violations == 0, rep.msg.decode()


def test_bad_arguments():
    mc = synth.CONFIGS["tiny"]
    cfg = B.make_config(mc)
    assert B.addr_check(cfg, 1, CUS, 0, [16], [1])[0] == B.MK_ERR_INVALID_ARG
    assert B.addr_check(cfg, 2, CUS, 1, [16, 16], [1, 1])[0] != 0   # batch > max_batch


@pytest.mark.parametrize("name,batch,steps", [("tiny", 1, 12), ("tiny_qk", 1, 8), ("tiny", 3, 8),
                                              ("tiny", 8, 4), ("llama1b", 1, 2), ("llama1b_b8", 8, 8)])
def test_one_launch_of_several_steps_in_bounds(name, batch, steps):
    """mk_decode_steps_greedy: the steps as one launch (logits row block per
    step, in-launch tokens, the token counter, positions + s); Llama-1B at
    batch 8 with 8 steps a launch is the benchmark's own launch."""
    mc = synth.CONFIGS[name]
    if batch > 1 and mc.batch != batch:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    mc = mc.replace(steps=steps)
    cfg = B.make_config(mc, max_batch=batch)
    rc, rep = B.addr_check(cfg, batch, CUS, steps, synth.make_positions(mc, batch),
                           synth.make_tokens(mc, batch), one_launch=True)
    assert rep.accesses > 0
    assert rc == 0 and rep.violations == 0, rep.msg.decode()


@pytest.mark.parametrize("batch", [1, 3])
def test_launch_logits_blocks_are_modelled(batch):
    """A logits buffer one row short: one step per launch writes its single
    row block, so the last row is reached at once; as one launch of several
    steps only the last step's last row falls outside, which the model must
    find (it would not if every step wrote the first row block)."""
    mc = synth.CONFIGS["tiny"]
    if batch > 1:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    mc = mc.replace(steps=4)
    cfg = B.make_config(mc, max_batch=batch)
    pos, tok = synth.make_positions(mc, batch), synth.make_tokens(mc, batch)
    rc, rep = B.addr_check(cfg, batch, CUS, 4, pos, tok, corrupt=6, one_launch=True)
    assert rc != 0 and rep.violations > 0 and "logits" in rep.msg.decode()
    rc, rep = B.addr_check(cfg, batch, CUS, 3, pos, tok, one_launch=True)
    assert rc == 0, rep.msg.decode()



@pytest.mark.parametrize("name,batch", [("tiny", 1), ("tiny_qk", 1), ("tiny", 3)])
@pytest.mark.parametrize("corrupt,sites", [(7, ("residual", "staged activation")), (8, ("tagged q",))])
def test_accesses_the_plan_does_not_record_are_found(name, batch, corrupt, sites):
    """The walk also checks every access to an activation buffer against the
    reads and writes the plan records for the unit (what the plan checker's
    dependency analysis sees): a plan that forgets the first FFN unit's
    residual read (7) or the first attention unit's tagged q/K/V read (8)
    must be reported where the kernel makes that access."""
    mc = synth.CONFIGS[name]
    if batch > 1:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    cfg = B.make_config(mc, max_batch=batch)
    rc, rep = B.addr_check(cfg, batch, CUS, 1, synth.make_positions(mc, batch), synth.make_tokens(mc, batch),
                           corrupt=corrupt)
    msg = rep.msg.decode()
    assert rc != 0 and "does not record" in msg and any(x in msg for x in sites), msg
