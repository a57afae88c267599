"""Seeded synthetic inputs for the Llama-style decode step.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It holds the workload shapes and draws the random tensors; it does no
arithmetic of the decode step itself (no norm, projection, rotation or
attention).  bf16 rounding of the drawn fp32 values is done by torch's own
conversion, a library routine.

Workloads (model shapes are those of a Llama-style pre-norm decoder; the
megakernel chapter "L'interpréteur sur GPU", section 3.1, quotes its latency
result on Llama-1B at batch 1):

* ``tiny``      2 layers, hidden 256, 4 query / 2 KV heads, head_dim 64,
                FFN 688, vocab 1024, 16 prior positions, batch 1.
* ``llama1b``   16 layers, hidden 2048, 32/8 heads, head_dim 64, FFN 8192,
                vocab 128256, tied embeddings, RoPE theta 5e5, 512 prior
                positions, batch 1, 32 greedy steps.
* ``llama1b_b8`` same shape, batch 8, positions per sequence uniform in
                [1024, 4096].
* ``qwen3_8b``  36 layers, hidden 4096, 32/8 heads, head_dim 128, per-head
                q/k RMSNorm, FFN 12288, vocab 151936, untied, 1024 prior.
* ``llama70b``  80 layers, hidden 8192, 64/8 heads, head_dim 128, FFN 28672,
                vocab 128256, untied, batch 64, 1024 prior.

Recipe: every tensor has its own ``numpy.random.SeedSequence([0, cfg_id,
kind, layer, idx])`` stream, drawn in C order.  Projection and embedding
weights are N(0, 0.02) rounded to bf16; norm weights are exactly 1.0; prior
KV slots are N(0, 1) rounded to bf16; tokens are uniform in [0, vocab).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

# Tensor kinds (part of each tensor's seed).
K_EMBED, K_LMHEAD, K_FINAL_NORM = 1, 2, 3
K_ATTN_NORM, K_WQ, K_WK, K_WV, K_QNORM, K_KNORM = 10, 11, 12, 13, 14, 15
K_WO, K_FFN_NORM, K_WGATE, K_WUP, K_WDOWN = 16, 17, 18, 19, 20
K_KV, K_TOKENS, K_POSITIONS = 30, 31, 32

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
              "ffn_norm", "w_gate", "w_up", "w_down")


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    cfg_id: int
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    tied_embeddings: bool = True
    qk_norm: bool = False
    batch: int = 1
    prior: int = 16            # prior positions for batch-1 workloads
    pos_lo: int = 0            # batched workloads: positions ~ U[pos_lo, pos_hi]
    pos_hi: int = 0
    steps: int = 32

    @property
    def max_seq(self) -> int:
        """KV capacity: the largest start position plus one slot per step."""
        start = self.pos_hi if self.batch > 1 and self.pos_hi else self.prior
        return start + self.steps

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)

    def weight_bytes(self) -> int:
        """bf16 bytes of every weight tensor read once per step."""
        H, F, hd = self.hidden, self.ffn_dim, self.head_dim
        q, kv = self.n_q_heads * hd, self.n_kv_heads * hd
        per_layer = (q + 2 * kv) * H + H * q + 3 * F * H + 2 * H
        if self.qk_norm:
            per_layer += 2 * hd
        head = self.vocab * H + H
        return 2 * (self.n_layers * per_layer + head)


CONFIGS: Dict[str, ModelConfig] = {
    "tiny": ModelConfig("tiny", 1, 2, 256, 4, 2, 64, 688, 1024,
                        rope_theta=10000.0, prior=16),
    "llama1b": ModelConfig("llama1b", 2, 16, 2048, 32, 8, 64, 8192, 128256,
                           rope_theta=500000.0, prior=512),
    "llama1b_b8": ModelConfig("llama1b_b8", 3, 16, 2048, 32, 8, 64, 8192,
                              128256, rope_theta=500000.0, batch=8,
                              pos_lo=1024, pos_hi=4096),
    "qwen3_8b": ModelConfig("qwen3_8b", 4, 36, 4096, 32, 8, 128, 12288,
                            151936, rope_theta=1000000.0,
                            tied_embeddings=False, qk_norm=True, prior=1024),
    "llama70b": ModelConfig("llama70b", 5, 80, 8192, 64, 8, 128, 28672,
                            128256, rope_theta=500000.0,
                            tied_embeddings=False, batch=64, prior=1024),
    # small parity case of the Qwen3 path: head_dim 128, q/k norm, untied
    "tiny_qk": ModelConfig("tiny_qk", 6, 2, 256, 4, 2, 128, 688, 1024,
                           rope_theta=1000000.0, tied_embeddings=False,
                           qk_norm=True, prior=16),
}


def _rng(cfg: ModelConfig, kind: int, layer: int = 0, idx: int = 0):
    return np.random.default_rng(
        np.random.SeedSequence([0, cfg.cfg_id, kind, layer, idx]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) through torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(cfg: ModelConfig, shape, std: float, kind: int,
                layer: int = 0, idx: int = 0) -> np.ndarray:
    g = _rng(cfg, kind, layer, idx)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x)


def ones_bf16(n: int) -> np.ndarray:
    return np.full((n,), 0x3F80, dtype=np.uint16)   # bf16 bits of 1.0


def _layer_shapes(cfg: ModelConfig):
    H, hd, F = cfg.hidden, cfg.head_dim, cfg.ffn_dim
    return {
        "wq": ((cfg.n_q_heads * hd, H), K_WQ),
        "wk": ((cfg.n_kv_heads * hd, H), K_WK),
        "wv": ((cfg.n_kv_heads * hd, H), K_WV),
        "wo": ((H, cfg.n_q_heads * hd), K_WO),
        "w_gate": ((F, H), K_WGATE),
        "w_up": ((F, H), K_WUP),
        "w_down": ((H, F), K_WDOWN),
    }


def make_weights(cfg: ModelConfig, std: float = 0.02,
                 threads: int = 8) -> dict:
    """All weights as bf16 bit arrays (numpy uint16), row-major [out][in].

    Returns ``{"embed", "final_norm", "lm_head" (None when tied), "layers":
    [ {attn_norm, wq, wk, wv, q_norm, k_norm, wo, ffn_norm, w_gate, w_up,
    w_down} ]}``; q_norm/k_norm are None unless the config has q/k norm.
    """
    H, hd = cfg.hidden, cfg.head_dim
    jobs = [("embed", None, (cfg.vocab, H), K_EMBED, 0)]
    if not cfg.tied_embeddings:
        jobs.append(("lm_head", None, (cfg.vocab, H), K_LMHEAD, 0))
    for l in range(cfg.n_layers):
        for key, (shape, kind) in _layer_shapes(cfg).items():
            jobs.append((key, l, shape, kind, l))

    def run(job):
        key, l, shape, kind, layer = job
        return job, normal_bf16(cfg, shape, std, kind, layer)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        results = list(ex.map(run, jobs))

    W = {"embed": None, "lm_head": None, "final_norm": ones_bf16(H),
         "layers": [dict(attn_norm=ones_bf16(H), ffn_norm=ones_bf16(H),
                         q_norm=ones_bf16(hd) if cfg.qk_norm else None,
                         k_norm=ones_bf16(hd) if cfg.qk_norm else None)
                    for _ in range(cfg.n_layers)]}
    for (key, l, _shape, _kind, _layer), arr in results:
        if l is None:
            W[key] = arr
        else:
            W["layers"][l][key] = arr
    return W


def make_kv_cache(cfg: ModelConfig, batch: Optional[int] = None,
                  max_seq: Optional[int] = None,
                  filled: Optional[int] = None) -> np.ndarray:
    """bf16 KV cache ``[L][2][B][n_kv][S][hd]`` with slots < ``filled``
    holding seeded N(0, 1) values and the rest zero."""
    B = cfg.batch if batch is None else batch
    S = cfg.max_seq if max_seq is None else max_seq
    n = S if filled is None else min(filled, S)
    kv = np.zeros((cfg.n_layers, 2, B, cfg.n_kv_heads, S, cfg.head_dim),
                  dtype=np.uint16)
    for l in range(cfg.n_layers):
        for t in range(2):
            blk = normal_bf16(cfg, (B, cfg.n_kv_heads, n, cfg.head_dim), 1.0,
                              K_KV, l, t)
            kv[l, t, :, :, :n, :] = blk
    return kv


def make_tokens(cfg: ModelConfig, batch: Optional[int] = None,
                step: int = 0) -> np.ndarray:
    B = cfg.batch if batch is None else batch
    return _rng(cfg, K_TOKENS, 0, step).integers(
        0, cfg.vocab, size=B, dtype=np.int64).astype(np.int32)


def make_positions(cfg: ModelConfig, batch: Optional[int] = None) -> np.ndarray:
    """Slot index of the new token per sequence (slots < p are prior)."""
    B = cfg.batch if batch is None else batch
    if cfg.pos_hi:
        return _rng(cfg, K_POSITIONS).integers(
            cfg.pos_lo, cfg.pos_hi + 1, size=B, dtype=np.int64).astype(np.int32)
    return np.full((B,), cfg.prior, dtype=np.int32)


def zero_like_layers(W: dict, keys: List[str]) -> dict:
    """Copy of ``W`` with the named per-layer tensors set to bf16 zero."""
    out = dict(W)
    out["layers"] = []
    for lw in W["layers"]:
        d = dict(lw)
        for k in keys:
            if d.get(k) is not None:
                d[k] = np.zeros_like(d[k])
        out["layers"].append(d)
    return out
