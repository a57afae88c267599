"""Plain CPU oracle of one Llama-style decode step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import or run this module.  It shares no code,
header, table or constant generator with the GPU path: it is written from
the pages, in numpy, slowly and in the order the definitions state.

What it computes.  The megakernel chapter ("L'interpréteur sur GPU", section
3.2, the table of seven fused instructions) names the work of one forward pass
of a Llama decoder: RMSNorm + QKV + RoPE, attention, attention reduction,
O-projection + residual, RMSNorm + up/gate + SiLU, down-projection + residual,
RMSNorm + LM head.  The pages never write the math of those steps down; the
plainest reading is the standard pre-norm Llama decoder, which this module
spells out.  The megakernel is an exact reorganisation of that forward pass
(index page "Partie 8", one-sentence definition: one persistent kernel runs
the whole model, kernel boundaries become counters), and its split attention
is mathematically identical to plain attention (GPU-kernels primer,
FlashAttention paragraph).  So the oracle is the plain definition.

Readings where the pages are silent:
  * RMSNorm: x * w / sqrt(mean(x^2) + eps), eps inside the root, weight after.
  * RoPE: half-split pairs (i, i + hd/2), angle p * theta^(-2i/hd), evaluated
    in float64 and rounded to float32 (cos and sin tables).
  * The KV cache holds post-RoPE K.  The new token's K and V are rounded to
    bf16 (round to nearest even) and written to slot p before attention, so
    the token attends to its own rounded K/V over slots 0..p inclusive.
  * Attention scale 1/sqrt(hd); GQA groups are contiguous heads.
  * SiLU(z) = z / (1 + exp(-z)); no biases; logits in float32.
  * q/k norm (only for models that have it): per head over hd, after the
    projection and before RoPE.
  * Everything else is carried in ``dt`` (float32 by default; float64 for
    tighter pins).

Pins (tests/test_oracle_*.py, all CPU): exhaustive bf16 decode/encode against
torch's conversion; matvec against float64 brute force within the textbook
bound; RMSNorm closed forms; RoPE against the complex-exponential form, norm
preservation, identity at p = 0, relative-position invariance; attention
single-key, identical-keys, shift invariance, split/LSE combine over any
partition; SiLU odd-part identity; model-level closed form with zeroed
weights, decode-equals-causal-prefill, batch independence, KV-slot
isolation.  No function here is left unpinned.
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "linear", "rmsnorm", "rope_cos_sin",
    "rope", "attention", "attention_partial", "attention_combine", "silu",
    "upcast_weights", "decode_step", "greedy", "generate",
]


# --------------------------------------------------------------------------
# bf16 <-> fp32.  The weights are 16-bit (chapter 3, section 3.1: a 16-bit
# model of more than a billion parameters); the KV cache is bf16.

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32, exact: the 16 bits are the top half of
    the float32 word."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    The kept 16 bits are the top half; the dropped half is compared with
    0x8000 and a tie rounds toward an even kept half.  NaN stays NaN (quiet).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    r = (hi + up.astype(np.uint64)) & np.uint64(0xFFFF)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, (hi | np.uint64(0x0040)) & np.uint64(0xFFFF), r)
    return r.astype(np.uint16)


def _f(a, dt):
    """A weight as ``dt``: bf16 bits are decoded, floats are cast."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = bf16_to_f32(a)
    return a.astype(dt, copy=False)


# --------------------------------------------------------------------------
# Elementary steps.

def linear(W, x, dt=np.float32) -> np.ndarray:
    """y = W x for W [out][in] (bf16 bits or float), x [in] or [B][in]."""
    Wf = _f(W, dt)
    xf = np.asarray(x, dtype=dt)
    return xf @ Wf.T if xf.ndim == 2 else Wf @ xf


def rmsnorm(x, w, eps: float, dt=np.float32) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w."""
    xf = np.asarray(x, dtype=dt)
    ms = np.mean(xf * xf, axis=-1, keepdims=True, dtype=dt)
    return (xf / np.sqrt(ms + dt(eps))) * _f(w, dt)


def rope_cos_sin(p: int, hd: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of the RoPE angles p * theta^(-2i/hd), i < hd/2.

    Angles are formed in float64 and the results rounded to float32."""
    i = np.arange(hd // 2, dtype=np.float64)
    ang = float(p) * np.power(float(theta), -2.0 * i / float(hd))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope(u, cos, sin, dt=np.float32) -> np.ndarray:
    """Rotate each pair (u_i, u_{i+hd/2}) of the last axis by its angle."""
    u = np.asarray(u, dtype=dt)
    h = u.shape[-1] // 2
    a, b = u[..., :h], u[..., h:]
    c, s = np.asarray(cos, dtype=dt), np.asarray(sin, dtype=dt)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q, K, V, dt=np.float32) -> np.ndarray:
    """Softmax attention of query rows q [G][hd] over keys K [T][hd] and
    values V [T][hd]; scale 1/sqrt(hd), maximum subtracted before exp."""
    q = np.asarray(q, dtype=dt)
    K = np.asarray(K, dtype=dt)
    V = np.asarray(V, dtype=dt)
    s = (q @ K.T) * dt(1.0 / math.sqrt(q.shape[-1]))
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    w = e / np.sum(e, axis=-1, keepdims=True)
    return w @ V


def attention_partial(q, K, V, dt=np.float32):
    """One split's (m, l, o): running max, sum of exp(s - m) and the
    unnormalised weighted sum of V, over the keys of the split.  An empty
    split gives (-inf, 0, 0).  This is the tiled/online-softmax form the
    attention step may be split into (chapter 3, instructions 2 and 3;
    FlashAttention paragraph of the GPU-kernels primer)."""
    q = np.asarray(q, dtype=dt)
    G, hd = q.shape
    if len(K) == 0:
        return (np.full(G, -np.inf, dtype=dt), np.zeros(G, dtype=dt),
                np.zeros((G, hd), dtype=dt))
    s = (q @ np.asarray(K, dtype=dt).T) * dt(1.0 / math.sqrt(hd))
    m = np.max(s, axis=-1)
    e = np.exp(s - m[:, None])
    return m, e.sum(axis=-1, dtype=dt), e @ np.asarray(V, dtype=dt)


def attention_combine(parts, dt=np.float32) -> np.ndarray:
    """Log-sum-exp combine of split partials into normalised attention
    output; empty splits (m = -inf) carry no weight."""
    ms = np.stack([p[0] for p in parts])            # [S][G]
    mstar = np.max(ms, axis=0)
    num = 0
    den = 0
    for m, l, o in parts:
        w = np.where(np.isneginf(m), dt(0), np.exp(np.where(
            np.isneginf(m), mstar, m) - mstar)).astype(dt)
        num = num + w[:, None] * o
        den = den + w * l
    return (num / den[:, None]).astype(dt)


def silu(z, dt=np.float32) -> np.ndarray:
    z = np.asarray(z, dtype=dt)
    return z / (dt(1) + np.exp(-z))


# --------------------------------------------------------------------------
# The decode step.

def upcast_weights(W: dict, dt=np.float32) -> dict:
    """Decode every bf16 tensor of ``W`` once (a convenience for repeated
    steps; the arithmetic is unchanged)."""
    up = lambda a: None if a is None else _f(a, dt)
    return {"embed": up(W["embed"]), "lm_head": up(W.get("lm_head")),
            "final_norm": up(W["final_norm"]),
            "layers": [{k: up(v) for k, v in lw.items()} for lw in W["layers"]]}


def decode_step(cfg, W: dict, tokens, positions, kv: np.ndarray,
                dt=np.float32, trace: Optional[dict] = None) -> np.ndarray:
    """One decode step for every sequence b < len(tokens).

    ``kv`` is the bf16 cache ``[L][2][B][n_kv][S][hd]`` (uint16 bits) and is
    updated in place at slot ``positions[b]`` of every layer.  Returns the
    float32 logits ``[B][vocab]``.  If ``trace`` is a dict it receives the
    per-layer intermediates (for stage-by-stage comparison).
    """
    H, hd = cfg.hidden, cfg.head_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    G = nq // nkv
    eps = cfg.rms_eps
    tokens = np.asarray(tokens)
    positions = np.asarray(positions)
    B = len(tokens)
    emb = W["embed"]
    h = np.stack([_f(emb[int(t)], dt) for t in tokens])          # [B][H]
    if trace is not None:
        trace.setdefault("h_in", []).append(h.copy())
    for l, lw in enumerate(W["layers"]):
        # Instruction 1: RMSNorm + QKV (+ q/k norm) + RoPE, K/V into the cache.
        x = rmsnorm(h, lw["attn_norm"], eps, dt)
        q = linear(lw["wq"], x, dt).reshape(B, nq, hd)
        k = linear(lw["wk"], x, dt).reshape(B, nkv, hd)
        v = linear(lw["wv"], x, dt).reshape(B, nkv, hd)
        if trace is not None:
            trace.setdefault("q_raw", []).append(q.copy())
        if cfg.qk_norm:
            q = rmsnorm(q, lw["q_norm"], eps, dt)
            k = rmsnorm(k, lw["k_norm"], eps, dt)
        attn = np.zeros((B, nq * hd), dtype=dt)
        qr_all = np.zeros((B, nq, hd), dtype=dt)
        for b in range(B):
            p = int(positions[b])
            c, s = rope_cos_sin(p, hd, cfg.rope_theta)
            qr = rope(q[b], c, s, dt)
            kr = rope(k[b], c, s, dt)
            qr_all[b] = qr
            kv[l, 0, b, :, p, :] = f32_to_bf16(kr.astype(np.float32))
            kv[l, 1, b, :, p, :] = f32_to_bf16(v[b].astype(np.float32))
            # Instructions 2 and 3: attention over slots 0..p of the cache.
            for g in range(nkv):
                Kg = bf16_to_f32(kv[l, 0, b, g, :p + 1, :])
                Vg = bf16_to_f32(kv[l, 1, b, g, :p + 1, :])
                o = attention(qr[g * G:(g + 1) * G], Kg, Vg, dt)
                attn[b, g * G * hd:(g + 1) * G * hd] = o.reshape(-1)
        # Instruction 4: O projection + residual.
        h_mid = h + linear(lw["wo"], attn, dt)
        # Instruction 5: RMSNorm + gate/up + SiLU.
        x2 = rmsnorm(h_mid, lw["ffn_norm"], eps, dt)
        a = silu(linear(lw["w_gate"], x2, dt), dt) * linear(lw["w_up"], x2, dt)
        # Instruction 6: down projection + residual.
        h_out = h_mid + linear(lw["w_down"], a, dt)
        if trace is not None:
            trace.setdefault("q", []).append(qr_all)
            trace.setdefault("attn", []).append(attn)
            trace.setdefault("h_mid", []).append(h_mid)
            trace.setdefault("a", []).append(a)
            trace.setdefault("h_out", []).append(h_out)
        h = h_out
    # Instruction 7: final RMSNorm + LM head (the embedding when tied).
    head = W["embed"] if cfg.tied_embeddings else W["lm_head"]
    xf = rmsnorm(h, W["final_norm"], eps, dt)
    return linear(head, xf, dt).astype(np.float32)


def greedy(logits) -> np.ndarray:
    """Next token per row: the arg max, lowest index on exact ties."""
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int32)


def generate(cfg, W, tokens, positions, kv, steps: int, dt=np.float32,
             force: Optional[List[np.ndarray]] = None):
    """``steps`` greedy decode steps.  Returns (tokens fed, logits) per step.

    ``force[i]``, if given, replaces the greedy choice fed to step i + 1
    (teacher forcing, for comparing runs after a near-tie)."""
    fed, outs = [], []
    tok = np.asarray(tokens, dtype=np.int32).copy()
    pos = np.asarray(positions, dtype=np.int32).copy()
    for i in range(steps):
        fed.append(tok.copy())
        lg = decode_step(cfg, W, tok, pos, kv, dt)
        outs.append(lg)
        tok = greedy(lg) if force is None else np.asarray(force[i], np.int32)
        pos = pos + 1
    return fed, outs
