"""Host-side pieces of bench.py: the overhead formula of the megakernels
chapter on when not to build one (section 9.1), pinned to the two recoveries
the section prints, the algorithmic byte count, and the stored-traffic
lookup."""
import json
import os

import pytest

import bench
from persistent_interpreter_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "overhead_examples.json")


def _golden():
    with open(GOLD) as f:
        return json.load(f)


def test_overhead_definition():
    assert bench.overhead(2.0, 1.0) == pytest.approx(0.5)
    assert bench.overhead(1.0, 1.0) == 0.0


def test_mpk_recovery_matches_printed_value():
    g = _golden()["mpk_qwen3_8b_a100"]
    r = bench.recovered(g["t_before_ms"], g["t_after_ms"], g["t_min_ms"])
    assert round(r, g["printed_digits"]) == g["recovered_printed"]


def test_hazy_recovery_matches_printed_value():
    g = _golden()["hazy_llama_1b"]
    r = bench.overhead_drop(g["bw_frac_before"], g["bw_frac_after"])
    assert round(r, g["printed_digits"]) == g["overhead_drop_printed"]


def test_algorithmic_bytes_llama1b():
    mc = synth.CONFIGS["llama1b"]
    # weights (bf16) + one embedding row + K and V of slots 0..512, 16 layers
    w = 2 * (mc.vocab * mc.hidden + mc.hidden
             + mc.n_layers * (2 * mc.hidden
                              + mc.hidden * (mc.n_q_heads + 2 * mc.n_kv_heads) * mc.head_dim
                              + mc.n_q_heads * mc.head_dim * mc.hidden
                              + 3 * mc.hidden * mc.ffn_dim))
    kv = 2 * 2 * mc.n_layers * mc.n_kv_heads * mc.head_dim * 513
    assert bench.algorithmic_bytes(mc, [512]) == w + 2 * mc.hidden + kv
    assert 2.4884e9 < bench.algorithmic_bytes(mc, [512]) < 2.4885e9  # 2,488.4 MB


def test_stored_traffic_only_for_matching_sources(monkeypatch):
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.stored_traffic("llama1b") is None
    assert bench.stored_traffic("no_such_workload") is None


def test_algorithmic_bytes_count_weights_once_per_step():
    """At batch B the step's algorithmic bytes add only each extra
    sequence's embedding row and K/V slots: the weights are read once per
    step whatever the batch (the batch-8 roofline prices against that)."""
    mc = synth.CONFIGS["llama1b_b8"]
    one = bench.algorithmic_bytes(mc, [2000])
    eight = bench.algorithmic_bytes(mc, [2000] * 8)
    kv_row = 2 * 2 * mc.n_layers * mc.n_kv_heads * mc.head_dim  # K and V bf16, one slot
    assert eight - one == 7 * (2 * mc.hidden + kv_row * 2001)
    assert one - bench.algorithmic_bytes(mc, [1999]) == kv_row
    assert bench.algorithmic_bytes(mc, []) == mc.weight_bytes()


def test_cpu_baseline_repeats_the_run_and_compares_the_first_pass():
    """The oracle leg on the tiny shape, with the oracle's own tokens and
    logits standing in for the GPU's: the first pass matches exactly, and
    the run repeats until the minimum time is reached."""
    import oracle as O
    from persistent_interpreter_amd import synth
    mc = synth.CONFIGS["tiny"].replace(steps=4)
    W = synth.make_weights(mc)
    kv0 = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    fed, lg = O.generate(mc, O.upcast_weights(W), tok, pos, kv0.copy(), 4)
    cpu, parity = bench.cpu_baseline(mc, W, kv0, tok, pos, fed, lg, min_s=0.3, budget_s=5.0)
    assert parity == {"max_abs_dlogit": 0.0, "greedy_match": "4/4"}
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    n = int(cpu["sample"].split()[0])
    assert n >= 8 and n % 4 == 0            # whole passes over the 4 steps
