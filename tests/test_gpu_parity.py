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


def _kv_bad(a, b, split_k=0):
    """Elements of two bf16 KV caches that differ by more than one bf16 ulp
    of the larger magnitude plus the arithmetic's own error.

    fp32 activations (batch 1): fp32 noise, 1e-4 of the RMS of the values
    that differ; the two sides round fp32 values computed in different
    orders, so a value near a rounding boundary, or near zero, may land one
    ulp (or a sign) apart.

    bf16 hi + lo activations (the batched MFMA path, ``split_k`` = the
    projection's K): each activation x enters as hi + lo with
    |x - hi - lo| <= 2^-16 |x| (two 8-bit mantissas), so a K-term projection
    moves by at most 2^-16 sum|w_i x_i|, which for random signs is about
    2^-16 sqrt(K) times the RMS of the outputs; the bar takes twice that."""
    fa = O.bf16_to_f32(a).astype(np.float64)
    fb = O.bf16_to_f32(b).astype(np.float64)
    d = np.abs(fa - fb)
    mag = np.maximum(np.abs(fa), np.abs(fb))
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
    if split_k:
        slack = 2.0 ** -15 * np.sqrt(split_k) * float(np.sqrt(np.mean(fb ** 2)))
    else:
        slack = 1e-4 * (float(np.sqrt(np.mean(fb[d > 0] ** 2))) if np.any(d > 0) else 1.0)
    bad = d > ulp + slack
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, d, -1)), d.shape)
        print(f"  worst KV element {tuple(int(x) for x in i)}: {fa[i]!r} vs {fb[i]!r}, "
              f"ulp {ulp[i]:.3e}, slack {slack:.3e}")
    return int(bad.sum()), float(d.max()) if d.size else 0.0


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


QK_SKIP = pytest.mark.skip(reason="q/k-norm path switched off: a 32-step run of it faulted "
                                   "the GPU; cause not found yet (the library returns "
                                   "MK_ERR_UNSUPPORTED for q/k norm)")


@pytest.mark.parametrize("name", ["tiny", pytest.param("tiny_qk", marks=QK_SKIP)])
def test_tiny_one_step_stages_and_logits(name):
    """Stage by stage against the oracle's intermediates.  With q/k norm the
    q buffer holds the raw projection (the attention units norm and rotate
    it), so it is compared with the oracle's projection output."""
    mc, W, sess, lg, ref, ref_kv, trace, tok, pos = _run_one(name)
    qref = trace["q_raw"] if mc.qk_norm else trace["q"]
    L, H, F = mc.n_layers, mc.hidden, mc.ffn_dim
    hb = sess.buffer(1, (2 * L + 1, 1, H))
    ab = sess.buffer(4, (L, 1, F))
    qb = sess.buffer(2, (L, 1, mc.n_q_heads, mc.head_dim))
    att = sess.buffer(3, (L, 1, mc.n_q_heads * mc.head_dim))
    for l in range(L):
        print(f"layer {l}: q {np.abs(qb[l] - qref[l]).max():.2e} "
              f"attn {np.abs(att[l] - trace['attn'][l]).max():.2e} "
              f"h_mid {np.abs(hb[2*l+1] - trace['h_mid'][l]).max():.2e} "
              f"a {np.abs(ab[l] - trace['a'][l]).max():.2e} "
              f"h_out {np.abs(hb[2*l+2] - trace['h_out'][l]).max():.2e}")
        np.testing.assert_allclose(qb[l], qref[l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(att[l], trace["attn"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(hb[2 * l + 1], trace["h_mid"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(ab[l], trace["a"][l], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(hb[2 * l + 2], trace["h_out"][l], atol=1e-4, rtol=1e-4)
    d = np.abs(lg - ref).max()
    print("tiny max |dlogit|", d)
    assert d <= TOL
    assert np.array_equal(np.argmax(lg, -1), np.argmax(ref, -1))
    gkv = sess.kv_host()
    nbad, dmax = _kv_bad(gkv, ref_kv)
    assert nbad == 0, (nbad, dmax)
    others = np.delete(np.arange(gkv.shape[4]), int(pos[0]))
    assert np.array_equal(gkv[:, :, :, :, others], ref_kv[:, :, :, :, others])
    sess.close()


@pytest.mark.parametrize("name,steps", [("tiny", 32), pytest.param("tiny_qk", 32, marks=QK_SKIP),
                                        ("llama1b", 32)])
def test_greedy_tokens_identical(name, steps):
    """Greedy decoding: the oracle, teacher-forced on the GPU's tokens with
    its own KV cache, picks the same token at every step and its logits stay
    within TOL.  The K/V slot each step writes is checked one step at a time:
    slots before position p are never rewritten, so the GPU's final cache
    holds exactly the history step p read; the oracle reruns step p on that
    history and its slot must match the GPU's to one bf16 ulp."""
    mc = synth.CONFIGS[name]
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    sess = harness.Session(mc, W, kv.copy())
    fed_g, out_g = harness.greedy_run(sess, tok, pos, steps)
    gkv = sess.kv_host()
    sess.close()
    Wf = O.upcast_weights(W)
    ref_kv = kv.copy()
    worst, kv_bad, kv_worst = 0.0, 0, 0.0
    for i in range(steps):
        ref = O.decode_step(mc, Wf, fed_g[i], pos + i, ref_kv)
        d = float(np.abs(out_g[i] - ref).max())
        worst = max(worst, d)
        top2 = np.sort(ref[0])[-2:]
        assert d <= TOL, (i, d)
        assert np.argmax(out_g[i][0]) == np.argmax(ref[0]), (i, top2, d)
        hist = gkv.copy()
        O.decode_step(mc, Wf, fed_g[i], pos + i, hist)
        slot = int(pos[0]) + i
        nb, dm = _kv_bad(gkv[:, :, :, :, slot], hist[:, :, :, :, slot])
        kv_bad += nb
        kv_worst = max(kv_worst, dm)
    print(f"{name}: {steps} steps, worst max|dlogit| {worst:.3e}; written KV "
          f"slots: {kv_bad} beyond tolerance, max abs diff {kv_worst:.3e}")
    assert kv_bad == 0, (kv_bad, kv_worst)
    untouched = np.r_[0:int(pos[0]), int(pos[0]) + steps:gkv.shape[4]]
    assert np.array_equal(gkv[:, :, :, :, untouched], kv[:, :, :, :, untouched])


BATCHED = [("tiny", 2, 32), ("tiny", 3, 8), ("tiny", 8, 8),
           pytest.param("llama1b_b8", 8, 32, marks=pytest.mark.timeout(900))]


@pytest.mark.parametrize("name,batch,steps", BATCHED)
def test_batched_greedy_matches_oracle(name, batch, steps):
    """Several sequences per step in one launch (the batched kernel: MFMA
    projections on bf16 hi + lo activations), each at its own position: the
    logits of every sequence stay within TOL of the oracle's (teacher-forced
    on the GPU's tokens, on the GPU's own KV history), the greedy tokens
    agree, the K/V slot each sequence writes matches to one bf16 ulp plus
    the split's own error, and no other slot of the cache changes."""
    mc = synth.CONFIGS[name]
    if mc.batch != batch or not mc.pos_hi:
        mc = mc.replace(batch=batch, pos_lo=4, pos_hi=40)
    W = synth.make_weights(mc)
    kv = synth.make_kv_cache(mc)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    print(f"{name}: batch {batch}, positions {pos.tolist()}", flush=True)
    sess = harness.Session(mc, W, kv.copy(), batch=batch)
    fed_g, out_g = harness.greedy_run(sess, tok, pos, steps)
    gkv = sess.kv_host()
    sess.close()
    Wf = O.upcast_weights(W)
    work = gkv.copy()   # GPU history; each step's slots are re-derived by the oracle
    bidx = np.arange(batch)
    worst, kv_bad = 0.0, 0
    for i in range(steps):
        ref = O.decode_step(mc, Wf, fed_g[i], pos + i, work)
        d = float(np.abs(out_g[i] - ref).max())
        worst = max(worst, d)
        assert d <= TOL, (i, d)
        assert np.array_equal(np.argmax(out_g[i], -1), np.argmax(ref, -1)), i
        for b in range(batch):
            s = int(pos[b]) + i
            nb, _ = _kv_bad(gkv[:, :, b, :, s], work[:, :, b, :, s], split_k=mc.hidden)
            kv_bad += nb
            work[:, :, b, :, s] = gkv[:, :, b, :, s]
    print(f"{name} batch {batch}: {steps} steps, worst max|dlogit| {worst:.3e}, "
          f"KV slots beyond tolerance {kv_bad}")
    assert kv_bad == 0
    # every slot no sequence wrote is untouched
    written = np.zeros(gkv.shape[2:5:2], dtype=bool)  # [B][S]
    for b in bidx:
        written[b, int(pos[b]):int(pos[b]) + steps] = True
    keep = ~written
    for b in bidx:
        assert np.array_equal(gkv[:, :, b, :, keep[b]], kv[:, :, b, :, keep[b]]), b
