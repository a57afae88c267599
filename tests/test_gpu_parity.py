"""GPU parity of the megakernel against the CPU oracle (through the C ABI).

Bars: max |logit difference| <= 2e-2 (bf16 weights, fp32 accumulation),
identical greedy tokens over 32 steps, and the K/V slot written by each step
equal to the oracle's bf16 values (at most one bf16 ulp apart where the two
fp32 values straddle a rounding boundary)."""
import numpy as np
import pytest

import oracle as O
from persistent_interpreter_amd import harness, synth

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _kv_ulps(a, b):
    """Largest difference between two bf16 bit arrays, in bf16 ulps of the
    larger magnitude; differences below 1e-6 (fp32 rounding noise around a
    value near zero, which can even flip its sign) count as 0."""
    fa = O.bf16_to_f32(a).astype(np.float64)
    fb = O.bf16_to_f32(b).astype(np.float64)
    d = np.abs(fa - fb)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(fa), np.abs(fb)), 1e-30))) - 7)
    r = np.where(d <= 1e-6, 0.0, d / ulp)
    return float(r.max()) if r.size else 0.0


def _run_one(name, **over):
    mc = synth.CONFIGS[name].replace(**over) if over else synth.CONFIGS[name]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    ref_kv = kv.copy()
    trace = {}
    ref = O.decode_step(mc, W, tok, pos, ref_kv, trace=trace)
    sess = harness.Session(mc, W, kv)
    sess.set_inputs(tok, pos)
    sess.step_checked()
    lg = sess.logits.cpu().numpy()
    return mc, W, sess, lg, ref, ref_kv, trace, tok, pos


def test_tiny_one_step_stages_and_logits():
    mc, W, sess, lg, ref, ref_kv, trace, tok, pos = _run_one("tiny")
    L, H, F = mc.n_layers, mc.hidden, mc.ffn_dim
    hb = sess.buffer(1, (2 * L + 1, 1, H))
    ab = sess.buffer(4, (L, 1, F))
    qb = sess.buffer(2, (L, 1, mc.n_q_heads, mc.head_dim))
    att = sess.buffer(3, (L, 1, mc.n_q_heads * mc.head_dim))
    for l in range(L):
        print(f"layer {l}: q {np.abs(qb[l] - trace['q'][l]).max():.2e} "
              f"attn {np.abs(att[l] - trace['attn'][l]).max():.2e} "
              f"h_mid {np.abs(hb[2*l+1] - trace['h_mid'][l]).max():.2e} "
              f"a {np.abs(ab[l] - trace['a'][l]).max():.2e} "
              f"h_out {np.abs(hb[2*l+2] - trace['h_out'][l]).max():.2e}")
        np.testing.assert_allclose(qb[l], trace["q"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(att[l], trace["attn"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(hb[2 * l + 1], trace["h_mid"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(ab[l], trace["a"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(hb[2 * l + 2], trace["h_out"][l], atol=1e-4, rtol=1e-4)
    d = np.abs(lg - ref).max()
    print("tiny max |dlogit|", d)
    assert d <= TOL
    assert np.array_equal(np.argmax(lg, -1), np.argmax(ref, -1))
    gkv = sess.kv_host()
    assert _kv_ulps(gkv, ref_kv) <= 1
    others = np.delete(np.arange(gkv.shape[4]), int(pos[0]))
    assert np.array_equal(gkv[:, :, :, :, others], ref_kv[:, :, :, :, others])
    sess.close()


@pytest.mark.parametrize("name,steps", [("tiny", 32), ("llama1b", 32)])
def test_greedy_tokens_identical(name, steps):
    mc = synth.CONFIGS[name]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    sess = harness.Session(mc, W, kv.copy())
    fed_g, out_g = harness.greedy_run(sess, tok, pos, steps)
    Wf = O.upcast_weights(W)
    ref_kv = kv.copy()
    worst = 0.0
    for i in range(steps):
        ref = O.decode_step(mc, Wf, fed_g[i], pos + i, ref_kv)
        d = float(np.abs(out_g[i] - ref).max())
        worst = max(worst, d)
        top2 = np.sort(ref[0])[-2:]
        assert d <= TOL, (i, d)
        assert np.argmax(out_g[i][0]) == np.argmax(ref[0]), (i, top2, d)
    print(f"{name}: {steps} steps, worst max|dlogit| {worst:.3e}")
    assert _kv_ulps(sess.kv_host(), ref_kv) <= 1
    sess.close()
