"""Model-level pins of the oracle's decode step: closed forms with zeroed
weights, decode equals an independently written causal prefill, batch
independence, KV-slot isolation and GQA-as-repeated-MHA.  CPU only, tiny
shapes."""
import math

import numpy as np
import pytest

import oracle as O
from persistent_interpreter_amd import synth

TINY = synth.CONFIGS["tiny"]


def _small(**kw):
    base = dict(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2,
                head_dim=16, ffn_dim=96, vocab=50, prior=0, steps=8)
    base.update(kw)
    return TINY.replace(**base)


def _closed_form_logits(cfg, W, t):
    e = O.bf16_to_f32(W["embed"][t]).astype(np.float64)
    x = e / math.sqrt(np.mean(e * e) + cfg.rms_eps)
    head = W["embed"] if cfg.tied_embeddings else W["lm_head"]
    return O.bf16_to_f32(head).astype(np.float64) @ x


@pytest.mark.parametrize("zeroed", [
    ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"],
    ["wo", "w_down"],
])
def test_zeroed_layers_give_closed_form(zeroed):
    cfg = TINY
    W = synth.zero_like_layers(synth.make_weights(cfg), zeroed)
    kv = synth.make_kv_cache(cfg, filled=cfg.prior)
    tok = synth.make_tokens(cfg)
    pos = synth.make_positions(cfg)
    lg = O.decode_step(cfg, W, tok, pos, kv, np.float64)
    ref = _closed_form_logits(cfg, W, int(tok[0]))
    np.testing.assert_allclose(lg[0], ref.astype(np.float32), rtol=1e-6,
                               atol=1e-6)
    # tied embeddings: the input token's own logit is |E_t|^2 / sqrt(
    # |E_t|^2/H + eps) (sqrt(H)*|E_t| when eps -> 0) and is the largest
    # for this seed
    e = O.bf16_to_f32(W["embed"][int(tok[0])]).astype(np.float64)
    n2 = float(e @ e)
    own = n2 / math.sqrt(n2 / cfg.hidden + cfg.rms_eps)
    assert abs(lg[0][int(tok[0])] - own) < 1e-5 * own
    assert O.greedy(lg)[0] == tok[0]


def _prefill(cfg, W, toks):
    """Causal prefill of ``toks`` at positions 0..T-1 from an empty cache,
    written in matrix form with a mask (independent of the decode loop)."""
    dt = np.float64
    T, H, hd = len(toks), cfg.hidden, cfg.head_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    G = nq // nkv
    f = lambda a: O.bf16_to_f32(a).astype(dt)
    h = f(W["embed"][toks])                                   # [T][H]
    cs = [O.rope_cos_sin(t, hd, cfg.rope_theta) for t in range(T)]
    cos = np.stack([c for c, _ in cs])[:, None, :]
    sin = np.stack([s for _, s in cs])[:, None, :]
    mask = np.triu(np.full((T, T), -np.inf), 1)
    for lw in W["layers"]:
        x = O.rmsnorm(h, lw["attn_norm"], cfg.rms_eps, dt)
        q = (x @ f(lw["wq"]).T).reshape(T, nq, hd)
        k = (x @ f(lw["wk"]).T).reshape(T, nkv, hd)
        v = (x @ f(lw["wv"]).T).reshape(T, nkv, hd)
        if cfg.qk_norm:
            q = O.rmsnorm(q, lw["q_norm"], cfg.rms_eps, dt)
            k = O.rmsnorm(k, lw["k_norm"], cfg.rms_eps, dt)
        q = O.rope(q, cos, sin, dt)
        k = O.rope(k, cos, sin, dt)
        kb = O.bf16_to_f32(O.f32_to_bf16(k.astype(np.float32))).astype(dt)
        vb = O.bf16_to_f32(O.f32_to_bf16(v.astype(np.float32))).astype(dt)
        out = np.zeros((T, nq, hd))
        for j in range(nq):
            s = q[:, j, :] @ kb[:, j // G, :].T / math.sqrt(hd) + mask
            s = np.exp(s - s.max(axis=1, keepdims=True))
            out[:, j, :] = (s / s.sum(axis=1, keepdims=True)) @ vb[:, j // G, :]
        h = h + out.reshape(T, nq * hd) @ f(lw["wo"]).T
        x2 = O.rmsnorm(h, lw["ffn_norm"], cfg.rms_eps, dt)
        g = x2 @ f(lw["w_gate"]).T
        a = g / (1 + np.exp(-g)) * (x2 @ f(lw["w_up"]).T)
        h = h + a @ f(lw["w_down"]).T
    head = W["embed"] if cfg.tied_embeddings else W["lm_head"]
    return O.rmsnorm(h, W["final_norm"], cfg.rms_eps, dt) @ f(head).T


@pytest.mark.parametrize("variant", [
    dict(), dict(qk_norm=True), dict(tied_embeddings=False),
    dict(n_kv_heads=4), dict(n_kv_heads=1)])
def test_decode_equals_causal_prefill(variant):
    cfg = _small(**variant)
    W = synth.make_weights(cfg, std=0.2)
    T = 7
    toks = np.random.default_rng(11).integers(0, cfg.vocab, T)
    ref = _prefill(cfg, W, toks)
    kv = synth.make_kv_cache(cfg, batch=1, max_seq=T, filled=0)
    for t in range(T):
        lg = O.decode_step(cfg, W, toks[t:t + 1], np.array([t]), kv, np.float64)
        np.testing.assert_allclose(lg[0], ref[t], rtol=1e-5, atol=1e-5)


def test_batch_rows_are_independent():
    cfg = _small(prior=5, steps=4)
    W = synth.make_weights(cfg, std=0.2)
    B = 3
    toks = np.array([3, 17, 42], dtype=np.int32)
    pos = np.array([5, 0, 8], dtype=np.int32)
    kv = synth.make_kv_cache(cfg, batch=B, max_seq=12)
    kv_b = kv.copy()
    lg = O.decode_step(cfg, W, toks, pos, kv_b, np.float64)
    for b in range(B):
        kv1 = kv[:, :, b:b + 1].copy()
        lg1 = O.decode_step(cfg, W, toks[b:b + 1], pos[b:b + 1], kv1, np.float64)
        np.testing.assert_allclose(lg[b], lg1[0], rtol=1e-12, atol=1e-12)
        assert np.array_equal(kv_b[:, :, b:b + 1], kv1)


def test_kv_append_touches_only_slot_p():
    cfg = TINY
    W = synth.make_weights(cfg)
    kv = synth.make_kv_cache(cfg)
    before = kv.copy()
    pos = synth.make_positions(cfg)
    O.decode_step(cfg, W, synth.make_tokens(cfg), pos, kv)
    p = int(pos[0])
    diff = np.argwhere(kv != before)
    assert len(diff) > 0 and np.all(diff[:, 4] == p)
    others = np.delete(np.arange(kv.shape[4]), p)
    assert np.array_equal(kv[:, :, :, :, others], before[:, :, :, :, others])


def test_gqa_equals_mha_with_repeated_kv_heads():
    cfg = _small(n_kv_heads=2, prior=6)
    G = cfg.n_q_heads // cfg.n_kv_heads
    W = synth.make_weights(cfg, std=0.2)
    kv = synth.make_kv_cache(cfg, batch=1, max_seq=8)
    hd = cfg.head_dim
    # MHA model: KV head j is GQA head j // G (contiguous groups)
    mha = cfg.replace(n_kv_heads=cfg.n_q_heads)
    Wm = dict(W)
    Wm["layers"] = []
    for lw in W["layers"]:
        d = dict(lw)
        for key in ("wk", "wv"):
            blocks = lw[key].reshape(cfg.n_kv_heads, hd, cfg.hidden)
            d[key] = np.repeat(blocks, G, axis=0).reshape(-1, cfg.hidden)
        Wm["layers"].append(d)
    kvm = np.repeat(kv, G, axis=3)
    tok, pos = np.array([9]), np.array([6])
    a = O.decode_step(cfg, W, tok, pos, kv, np.float64)
    b = O.decode_step(mha, Wm, tok, pos, kvm, np.float64)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.repeat(kv, G, axis=3), kvm)


def test_fp32_oracle_close_to_fp64():
    cfg = TINY
    W = synth.make_weights(cfg)
    kv = synth.make_kv_cache(cfg)
    tok, pos = synth.make_tokens(cfg), synth.make_positions(cfg)
    a = O.decode_step(cfg, W, tok, pos, kv.copy(), np.float32)
    b = O.decode_step(cfg, W, tok, pos, kv.copy(), np.float64)
    assert np.max(np.abs(a - b)) < 1e-4


def test_qk_norm_makes_logits_invariant_to_scaling_wq_wk():
    """Per-head RMSNorm of q and k (Qwen3) removes any positive scale of the
    q/k projections (RMSNorm is scale invariant while |c|*rms >> sqrt(eps)):
    doubling Wq and Wk (exact in bf16) leaves the logits unchanged with q/k
    norm, and changes them without it."""
    for qk in (True, False):
        cfg = _small(qk_norm=qk)
        W = synth.make_weights(cfg, std=0.2)
        W2 = {**W, "layers": []}
        for lw in W["layers"]:
            lw2 = dict(lw)
            for name in ("wq", "wk"):
                f = O.bf16_to_f32(lw[name]) * 2.0        # exact: power of two
                lw2[name] = O.f32_to_bf16(f)
            W2["layers"].append(lw2)
        outs = []
        for WW in (W, W2):
            kv = synth.make_kv_cache(cfg, batch=1, max_seq=4, filled=0)
            for t in range(3):
                lg = O.decode_step(cfg, WW, np.array([5 + t]), np.array([t]), kv, np.float64)
            outs.append(lg)
        d = np.abs(outs[0] - outs[1]).max()
        scale = np.abs(outs[0]).max()
        if qk:   # float32 logits (a few ulps) and the eps inside the root
            assert d < 1e-5 * scale, (d, scale)
        else:    # scores grow four-fold
            assert d > 1e-2 * scale, (d, scale)


def _first_max_loop(row):
    """The arg max by a plain scan: the first index holding the largest
    value, where a NaN counts as larger than every number and the first NaN
    wins."""
    best, bi = None, -1
    for i, v in enumerate(row):
        if bi < 0:
            best, bi = v, i
        elif math.isnan(best):
            break
        elif math.isnan(v) or v > best:
            best, bi = v, i
    return bi


def test_greedy_lowest_index_on_exact_ties():
    """The greedy choice (reading: ties go to the lowest index) against a
    plain scan, on rows built with exact ties at the front, the back and in
    between, all-equal rows, -inf entries, signed zeros and NaN."""
    rng = np.random.default_rng(11)
    rows = [np.zeros(7, np.float32), np.full(5, -np.inf, np.float32),
            np.array([-0.0, 0.0, 0.0], np.float32),
            np.array([1.0, np.nan, 3.0, np.nan], np.float32)]
    for _ in range(200):
        n = int(rng.integers(1, 40))
        r = rng.integers(-3, 4, n).astype(np.float32)       # many exact ties
        if rng.random() < 0.3:
            r[rng.integers(0, n)] = -np.inf
        rows.append(r)
    for r in rows:
        got = int(O.greedy(r[None, :])[0])
        assert got == _first_max_loop(list(r)), r
    # a batch of rows is row by row
    B = np.stack([rng.integers(-2, 3, 16).astype(np.float32) for _ in range(6)])
    assert list(O.greedy(B)) == [_first_max_loop(list(b)) for b in B]
