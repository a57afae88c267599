"""Glue for tests, the bench and the smoke run: upload seeded inputs to the
GPU, own the step buffers, and drive greedy decoding through the C ABI.

Nothing here computes any part of the decode step: the step itself is one
``mk_decode_step`` launch.  The greedy choice of the next token (an argmax
over the logits the kernel wrote) and ``position + 1`` are harness work in
``advance_greedy``, or kernel work in ``step_greedy``
(``mk_decode_step_greedy``), which writes them over the step's own token and
position buffers so that steps chain on the device.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import binding as B
from . import synth


def _t(a: Optional[np.ndarray], device):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def upload_weights(W: dict, device="cuda") -> dict:
    """bf16 bit arrays -> device int16 tensors (same bits)."""
    return {"embed": _t(W["embed"], device), "final_norm": _t(W["final_norm"], device),
            "lm_head": _t(W.get("lm_head"), device),
            "layers": [{k: _t(v, device) for k, v in lw.items()} for lw in W["layers"]]}


class Session:
    """A megakernel handle plus device-resident step buffers."""

    def __init__(self, mc: synth.ModelConfig, W: dict, kv: np.ndarray,
                 batch: int = 1, device="cuda", **knobs):
        import torch
        self.mc = mc
        self.batch = batch
        self.device = device
        self.dW = upload_weights(W, device) if not _is_device(W) else W
        self.kv = _t(kv, device) if isinstance(kv, np.ndarray) else kv
        max_batch = kv.shape[2]
        max_seq = kv.shape[4]
        self.cfg = B.make_config(mc, max_batch=max_batch, max_seq=max_seq, **knobs)
        self.mk = B.Megakernel(self.cfg, self.dW)
        self.tokens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.positions = torch.zeros(batch, dtype=torch.int32, device=device)
        self.logits = torch.zeros(batch, mc.vocab, dtype=torch.float32, device=device)

    def set_inputs(self, tokens, positions):
        import torch
        self.tokens.copy_(torch.as_tensor(np.asarray(tokens, np.int32)))
        self.positions.copy_(torch.as_tensor(np.asarray(positions, np.int32)))

    def step(self) -> int:
        return self.mk.decode_step(self.batch, self.tokens, self.positions, self.kv, self.logits)

    def step_greedy(self) -> int:
        """One step that also replaces the tokens and positions with the
        greedy next token and position (in the same launch)."""
        return self.mk.decode_step_greedy(self.batch, self.tokens, self.positions, self.kv,
                                          self.logits, self.tokens, self.positions)

    def step_checked(self):
        rc = self.step()
        if rc != B.MK_OK:
            raise B.MkError(rc, "mk_decode_step")
        rc = self.mk.sync_status()
        if rc != B.MK_OK:
            raise B.MkError(rc, "device")

    def advance_greedy(self):
        """Feed the arg max of the last logits at the next position."""
        self.tokens.copy_(greedy_tokens(self.logits))
        self.positions.add_(1)

    def kv_host(self) -> np.ndarray:
        return self.kv.cpu().numpy().view(np.uint16)

    TAGGED = (2,)  # MK_BUF_Q holds (value, tag) words

    def buffer(self, which: int, shape, dtype=np.float32) -> np.ndarray:
        """Copy of one of the library's internal buffers (mk_get_buffer).
        Tagged buffers hold 64-bit words (fp32 value in the low half, the
        step's tag in the high half); their values are returned."""
        import ctypes
        import torch
        ptr, nbytes = self.mk.buffer(which)
        tagged = which in self.TAGGED
        out = np.empty(shape, dtype=np.uint64 if tagged else dtype)
        assert out.nbytes <= nbytes
        torch.cuda.synchronize()
        hip = ctypes.CDLL("libamdhip64.so")
        rc = hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(ptr),
                           ctypes.c_size_t(out.nbytes), 2)  # device to host
        assert rc == 0, rc
        if tagged:
            out = (out & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
        return out

    def close(self):
        self.mk.close()


def _chunks(V: int) -> int:
    """A divisor of V near sqrt(V) (1 if V has none between 16 and V / 16)."""
    best = 1
    for c in range(16, int(V ** 0.5) * 2 + 1):
        if V % c == 0 and V // c >= 16 and abs(c - V ** 0.5) < abs(best - V ** 0.5):
            best = c
    return best


def greedy_tokens(logits):
    """int32 arg max over the last axis of fp32 ``logits`` [B][V], first index
    on ties (as ``torch.argmax``), in two short reductions: the maximum of
    each of C chunks of V / C logits, then the first chunk holding the
    largest.  One reduction over all V logits of a row runs on few workgroups
    and takes several times longer on the GPU."""
    import torch
    B, V = logits.shape
    C = _chunks(V)
    if C == 1:
        return torch.argmax(logits, dim=-1).to(torch.int32)
    v, i = logits.view(B, C, V // C).max(dim=2)
    j = v.argmax(dim=1, keepdim=True)
    return (i.gather(1, j).squeeze(1) + j.squeeze(1) * (V // C)).to(torch.int32)


def _is_device(W) -> bool:
    return not isinstance(W.get("embed"), np.ndarray)


def greedy_run(sess: Session, tokens, positions, steps: int):
    """Run ``steps`` greedy steps; returns (fed tokens, logits) per step on
    the host."""
    sess.set_inputs(tokens, positions)
    fed: List[np.ndarray] = []
    outs: List[np.ndarray] = []
    for _ in range(steps):
        fed.append(sess.tokens.cpu().numpy().copy())
        sess.step_checked()
        outs.append(sess.logits.cpu().numpy().copy())
        sess.advance_greedy()
    return fed, outs
