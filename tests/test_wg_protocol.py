"""The ordering inside a workgroup of the batch-1 and batched kernels, on
the host (tests/wg_model.py): the library's own queues (mk_plan_units) run
through a model of the loader, sync and compute waves' LDS protocol under
random schedules with long stalls of single waves.  check_plan covers the ordering
between workgroups and mk_addr_check the addresses; this covers the
handshakes between the waves of one workgroup: page ring slots and their
sentinels, activation slots, result slots and the epilogue that frees them.

The model's sensitivity is pinned by planting protocol errors: each must be
caught on the same queues."""
import pytest

import wg_model as W
from persistent_interpreter_amd import binding as B, synth

CUS = 256


def _queues(name, batch=1):
    mc = synth.CONFIGS[name]
    units, q = B.plan_units(B.make_config(mc, max_batch=max(batch, mc.batch)), batch, CUS)
    return [units[q[c]:q[c + 1]] for c in range(CUS) if q[c + 1] > q[c]]


def test_plan_units_matches_the_report():
    mc = synth.CONFIGS["llama1b"]
    cfg = B.make_config(mc)
    units, q = B.plan_units(cfg, 1, CUS)
    rc, rep = B.plan_check(cfg, 1, CUS)
    assert rc == 0 and rep.n_instr == len(units) and q[-1] == len(units)
    assert sum(u.pages for u in units) == rep.n_pages
    ops = {u.op for u in units}
    assert ops == {W.OP_QKV, W.OP_ATTN, W.OP_RED, W.OP_O, W.OP_FFN, W.OP_DOWN, W.OP_LM}


@pytest.mark.parametrize("name", ["tiny", "llama1b"])
def test_queues_run_clean(name):
    """Every tiny queue and a spread of Llama-1B queues (first, middle,
    last workgroups, which hold different unit mixes), several schedules
    each."""
    qs = _queues(name)
    pick = qs if name == "tiny" else [qs[i] for i in (0, 1, 63, 128, 191, len(qs) - 1)]
    for i, qu in enumerate(pick):
        for seed in range(3):
            W.simulate(qu, seed=seed * 1000 + i)


def test_ring_of_fewer_pages_still_clean():
    """The protocol does not depend on the ring size: 4 and 5 pages."""
    qu = _queues("llama1b")[7]
    for p in (4, 5):
        W.simulate(qu, seed=p, ring_pages=p)


@pytest.mark.parametrize("knob,kw,what", [
    ("early_slot", {}, ("page", "deadlock")),
    ("early_xs", {}, ("activation piece",)),
    ("no_guard", {"nxs": 4}, ("result slot",)),
])
@pytest.mark.parametrize("name", ["tiny", "llama1b"])
def test_planted_protocol_errors_are_caught(name, knob, kw, what):
    qs = _queues(name)
    qu = max(qs[:8], key=len)
    caught = []
    for seed in range(8):
        try:
            W.simulate(qu, seed=seed, knobs=(knob,), budget=3_000_000, **kw)
        except W.ProtocolError as e:
            caught.append(str(e))
            break
    assert caught, f"{knob} was not caught on {name}"
    assert any(w in caught[0] for w in what), caught[0]


# ---- the batched kernel: six-page ring, four activation slots with three
# pieces in flight, MFMA tiles, two partial-tile buffers

@pytest.mark.parametrize("name,batch", [("tiny", 3), ("tiny", 8), ("llama1b_b8", 8)])
def test_batched_queues_run_clean(name, batch):
    qs = _queues(name, batch)
    pick = qs if name == "tiny" else [qs[i] for i in (0, 1, 63, 128, 191, len(qs) - 1)]
    for i, qu in enumerate(pick):
        for seed in range(2):
            W.simulate_batched(qu, seed=seed * 1000 + i)


def test_batched_ring_of_fewer_pages_still_clean():
    """A 16-row tile pair spans at most two pages, so 3 and 4 ring pages
    still let every wave finish."""
    qu = max(_queues("llama1b_b8", 8)[:8], key=len)
    for p in (3, 4):
        W.simulate_batched(qu, seed=p, ring_pages=p)


# Each plant is checked on a queue where it can bite.  With Llama-1B's four
# pieces per projection the activation-slot wait alone keeps the sync wave
# within one unit of the slowest compute wave, which already orders the
# result slots and partial-tile buffers; the tiny shape's one-piece units
# leave those guards as the only order.  Conversely, on the tiny shape the
# result-slot guard keeps the sync wave from reaching a slot still being
# read, so an early activation-slot release shows only on Llama-1B.
@pytest.mark.parametrize("name,batch,knob,what", [
    ("tiny", 3, "early_slot", ("page", "deadlock")),
    ("llama1b_b8", 8, "early_slot", ("page", "deadlock")),
    ("llama1b_b8", 8, "early_xs", ("activation piece",)),
    ("tiny", 3, "no_guard", ("result slot",)),
    ("tiny", 8, "no_part_guard", ("partial tile", "candidate area")),
])
def test_batched_planted_protocol_errors_are_caught(name, batch, knob, what):
    qu = max(_queues(name, batch)[:8], key=len)
    caught = []
    for seed in range(8):
        try:
            W.simulate_batched(qu, seed=seed, knobs=(knob,), budget=3_000_000)
        except W.ProtocolError as e:
            caught.append(str(e))
            break
    assert caught, f"{knob} was not caught on {name} batch {batch}"
    assert any(w in caught[0] for w in what), caught[0]
