"""ctypes binding of the C ABI in include/mk.h (argument marshalling only).

Every step of the decode path runs in the library's HIP kernel; this module
only converts Python/torch objects to pointers and sizes.  Loading fails
loudly if the library has not been built.
"""
from __future__ import annotations

import atexit
import ctypes as C
import os
import sys
import weakref
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# MK_LIB_PATH selects another build of the same library (a compile-time knob
# variant, for measurements); the default is the in-tree build.
LIB_PATH = os.environ.get("MK_LIB_PATH") or os.path.join(_HERE, "_lib", "libmk.so")

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_UNSUPPORTED = -2
MK_ERR_OOM = -3
MK_ERR_HIP = -4
MK_ERR_NOT_CORESIDENT = -5
MK_ERR_NO_DEVICE = -6
MK_ERR_NOT_PREPARED = -7
MK_ERR_DEVICE_TIMEOUT = -10
MK_ERR_BAD_TOKEN = -11
MK_ERR_BAD_POSITION = -12

MK_FLAG_TRACE = 1
MK_FLAG_COOPERATIVE = 2
MK_FLAG_PERTURB = 4
MK_FLAG_TEST_STALL = 8

MK_BUF_H, MK_BUF_Q, MK_BUF_ATTN, MK_BUF_A, MK_BUF_TRACE = 1, 2, 3, 4, 5

EXPORTED = ("mk_create", "mk_decode_step", "mk_decode_step_greedy",
            "mk_sync_status", "mk_destroy", "mk_strerror", "mk_plan_check",
            "mk_get_buffer", "mk_version", "mk_stream_read",
            "mk_stream_read_sink_words", "mk_addr_check",
            "mk_decode_step_static", "mk_decode_steps_greedy",
            "mk_addr_check_launch", "mk_plan_units")


class MkConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float), ("tied_embeddings", C.c_int32),
                ("qk_norm", C.c_int32), ("max_batch", C.c_int32),
                ("max_seq", C.c_int32), ("mlp_chunks", C.c_int32),
                ("kv_splits", C.c_int32), ("num_cus", C.c_int32),
                ("watchdog_ms", C.c_int32), ("flags", C.c_uint32)]


class MkLayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                 "ffn_norm", "w_gate", "w_up", "w_down")]


class MkWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p), ("layers", C.POINTER(MkLayerWeights))]


class MkPlanReport(C.Structure):
    _fields_ = [("num_cus", C.c_int32), ("batch", C.c_int32),
                ("kv_splits", C.c_int32), ("mlp_chunks", C.c_int32),
                ("n_instr", C.c_int32), ("n_groups", C.c_int32),
                ("n_pages", C.c_int32), ("max_queue", C.c_int32),
                ("weight_bytes", C.c_int64), ("max_cu_bytes", C.c_int64),
                ("mfma_cols_k", C.c_int64),
                ("sim_runs", C.c_int32), ("sim_errors", C.c_int32),
                ("paged_kv", C.c_int32), ("down_splits", C.c_int32),
                ("msg", C.c_char * 256)]


class MkUnitInfo(C.Structure):
    _fields_ = [("op", C.c_int32), ("layer", C.c_int32), ("nk", C.c_int32),
                ("pages", C.c_int32), ("ppp", C.c_int32), ("n_items", C.c_int32),
                ("ipw", C.c_int32), ("wait_n", C.c_int32), ("b", C.c_int32),
                ("aux0", C.c_int32), ("aux1", C.c_int32), ("split_len", C.c_int32)]


class MkAddrReport(C.Structure):
    _fields_ = [("accesses", C.c_int64), ("violations", C.c_int32),
                ("msg", C.c_char * 256)]


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m persistent_interpreter_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.mk_create.argtypes = [C.POINTER(MkConfig), C.POINTER(MkWeights),
                                C.POINTER(C.c_void_p)]
        L.mk_create.restype = C.c_int
        L.mk_decode_step.argtypes = [C.c_void_p, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p]
        L.mk_decode_step.restype = C.c_int
        L.mk_decode_step_greedy.argtypes = [C.c_void_p, C.c_int32, C.c_void_p,
                                            C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_void_p, C.c_void_p, C.c_void_p]
        L.mk_decode_step_greedy.restype = C.c_int
        L.mk_decode_steps_greedy.argtypes = [C.c_void_p, C.c_int32, C.c_int32,
                                             C.c_void_p, C.c_void_p, C.c_void_p,
                                             C.c_void_p, C.c_void_p, C.c_void_p,
                                             C.c_void_p]
        L.mk_decode_steps_greedy.restype = C.c_int
        L.mk_decode_step_static.argtypes = [C.c_void_p, C.c_int32, C.c_void_p,
                                            C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_void_p, C.c_void_p, C.c_void_p]
        L.mk_decode_step_static.restype = C.c_int
        L.mk_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
        L.mk_stream_read.restype = C.c_int
        L.mk_stream_read_sink_words.argtypes = []
        L.mk_stream_read_sink_words.restype = C.c_size_t
        L.mk_sync_status.argtypes = [C.c_void_p]
        L.mk_sync_status.restype = C.c_int
        L.mk_destroy.argtypes = [C.c_void_p]
        L.mk_destroy.restype = None
        L.mk_strerror.argtypes = [C.c_int]
        L.mk_strerror.restype = C.c_char_p
        L.mk_plan_check.argtypes = [C.POINTER(MkConfig), C.c_int32, C.c_int32,
                                    C.c_int32, C.c_int32, C.c_uint64,
                                    C.POINTER(MkPlanReport)]
        L.mk_plan_check.restype = C.c_int
        L.mk_get_buffer.argtypes = [C.c_void_p, C.c_int32,
                                    C.POINTER(C.c_void_p),
                                    C.POINTER(C.c_size_t)]
        L.mk_get_buffer.restype = C.c_int
        L.mk_plan_units.argtypes = [C.POINTER(MkConfig), C.c_int32, C.c_int32,
                                    C.POINTER(MkUnitInfo), C.c_int32, C.POINTER(C.c_int32)]
        L.mk_plan_units.restype = C.c_int
        L.mk_addr_check.argtypes = [C.POINTER(MkConfig), C.c_int32, C.c_int32,
                                    C.c_int32, C.POINTER(C.c_int32),
                                    C.POINTER(C.c_int32), C.c_int32,
                                    C.POINTER(MkAddrReport)]
        L.mk_addr_check.restype = C.c_int
        L.mk_addr_check_launch.argtypes = [C.POINTER(MkConfig), C.c_int32, C.c_int32,
                                    C.c_int32, C.POINTER(C.c_int32),
                                    C.POINTER(C.c_int32), C.c_int32,
                                    C.POINTER(MkAddrReport)]
        L.mk_addr_check_launch.restype = C.c_int
        L.mk_version.argtypes = []
        L.mk_version.restype = C.c_int
        _lib = L
    return _lib


class MkError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


def strerror(code: int) -> str:
    return lib().mk_strerror(code).decode()


def make_config(mc, max_batch: int = 1, max_seq: Optional[int] = None,
                mlp_chunks: int = 0, kv_splits: int = 0, num_cus: int = 0,
                watchdog_ms: int = 0, flags: int = 0) -> MkConfig:
    """MkConfig from a model-shape object (``synth.ModelConfig``)."""
    return MkConfig(mc.n_layers, mc.hidden, mc.n_q_heads, mc.n_kv_heads,
                    mc.head_dim, mc.ffn_dim, mc.vocab, mc.rms_eps,
                    mc.rope_theta, int(mc.tied_embeddings), int(mc.qk_norm),
                    max_batch, mc.max_seq if max_seq is None else max_seq,
                    mlp_chunks, kv_splits, num_cus, watchdog_ms, flags)


def plan_check(cfg: MkConfig, batch: int, num_cus: int, sim_runs: int = 0,
               corrupt: int = 0, seed: int = 0):
    rep = MkPlanReport()
    rc = lib().mk_plan_check(C.byref(cfg), batch, num_cus, sim_runs, corrupt,
                             seed, C.byref(rep))
    return rc, rep


def addr_check(cfg: MkConfig, batch: int, num_cus: int, steps: int,
               positions, tokens, corrupt: int = 0, one_launch: bool = False):
    """Run the host address model (mk_addr_check, or with one_launch
    mk_addr_check_launch: the steps as one launch); returns (rc, report)."""
    rep = MkAddrReport()
    pos = (C.c_int32 * batch)(*[int(x) for x in positions])
    tok = (C.c_int32 * batch)(*[int(x) for x in tokens])
    fn = lib().mk_addr_check_launch if one_launch else lib().mk_addr_check
    rc = fn(C.byref(cfg), batch, num_cus, steps, pos, tok, corrupt, C.byref(rep))
    return rc, rep


def plan_units(cfg: MkConfig, batch: int, num_cus: int):
    """The schedule's units (mk_plan_units): (list of MkUnitInfo, q_off)."""
    n = lib().mk_plan_units(C.byref(cfg), batch, num_cus, None, 0, None)
    if n < 0:
        raise MkError(n, "mk_plan_units")
    units = (MkUnitInfo * max(n, 1))()
    q_off = (C.c_int32 * (num_cus + 1))()
    rc = lib().mk_plan_units(C.byref(cfg), batch, num_cus, units, n, q_off)
    if rc != n:
        raise MkError(rc, "mk_plan_units")
    return list(units)[:n], list(q_off)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


# Every live handle, closed by an exit hook that runs before the interpreter
# tears down its modules (and long before the HIP runtime's own exit-time
# teardown), so mk_destroy never runs from a finalizer at shutdown.
_LIVE: "weakref.WeakSet" = weakref.WeakSet()


@atexit.register
def _close_all():
    for mk in list(_LIVE):
        mk.close()


class Megakernel:
    """Owns an ``mk_handle``.  ``weights`` maps names to device tensors
    (bf16 or int16 views of bf16 bits): embed, final_norm, lm_head (or None)
    and layers = list of dicts with the per-layer names of ``mk.h``."""

    def __init__(self, cfg: MkConfig, weights: dict):
        self.cfg = cfg
        self._keep = weights
        n = cfg.n_layers
        arr = (MkLayerWeights * n)()
        for l, lw in enumerate(weights["layers"]):
            for name, _ in MkLayerWeights._fields_:
                setattr(arr[l], name, _ptr(lw.get(name)))
        self._layers = arr
        w = MkWeights(_ptr(weights["embed"]), _ptr(weights["final_norm"]),
                      _ptr(weights.get("lm_head")),
                      C.cast(arr, C.POINTER(MkLayerWeights)))
        h = C.c_void_p()
        rc = lib().mk_create(C.byref(cfg), C.byref(w), C.byref(h))
        if rc != MK_OK:
            raise MkError(rc, "mk_create")
        self.h = h
        _LIVE.add(self)

    def decode_step(self, batch: int, tokens, positions, kv, logits,
                    stream: Optional[int] = None) -> int:
        """Enqueue one decode step; returns the synchronous status."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        return lib().mk_decode_step(self.h, batch, _ptr(tokens), _ptr(positions),
                                    _ptr(kv), _ptr(logits), stream)

    def decode_step_greedy(self, batch: int, tokens, positions, kv, logits,
                           next_tokens, next_positions,
                           stream: Optional[int] = None) -> int:
        """Enqueue one decode step that also writes the greedy next token and
        position (device int32 [batch] each; they may be `tokens` and
        `positions` themselves); returns the synchronous status."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        return lib().mk_decode_step_greedy(self.h, batch, _ptr(tokens), _ptr(positions),
                                           _ptr(kv), _ptr(logits), _ptr(next_tokens),
                                           _ptr(next_positions), stream)

    def decode_steps_greedy(self, batch: int, n_steps: int, tokens, positions, kv,
                            logits, next_tokens, next_positions,
                            stream: Optional[int] = None) -> int:
        """Enqueue n_steps chained greedy decode steps in one launch; logits
        is fp32 [n_steps][batch][vocab]; returns the synchronous status."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        return lib().mk_decode_steps_greedy(self.h, batch, n_steps, _ptr(tokens),
                                            _ptr(positions), _ptr(kv), _ptr(logits),
                                            _ptr(next_tokens), _ptr(next_positions), stream)

    def decode_step_static(self, batch: int, tokens, positions, kv, logits,
                           next_tokens=None, next_positions=None,
                           stream: Optional[int] = None) -> int:
        """mk_decode_step_static: the step on the library's static scratch
        (no allocation); the batch size's schedule must already exist."""
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        return lib().mk_decode_step_static(self.h, batch, _ptr(tokens), _ptr(positions),
                                           _ptr(kv), _ptr(logits), _ptr(next_tokens),
                                           _ptr(next_positions), stream)

    def sync_status(self) -> int:
        return lib().mk_sync_status(self.h)

    def plan_splits(self, batch: int) -> int:
        """KV splits of this handle's plan for `batch` (host-side planner)."""
        rc, rep = plan_check(self.cfg, batch, 256)
        return int(rep.kv_splits) if rc == MK_OK else -1

    def buffer(self, which: int):
        p, n = C.c_void_p(), C.c_size_t()
        rc = lib().mk_get_buffer(self.h, which, C.byref(p), C.byref(n))
        if rc != MK_OK:
            raise MkError(rc, "mk_get_buffer")
        return p.value, n.value

    def close(self):
        """Free the handle (synchronising the device first, so no step of it
        is still running when its buffers go)."""
        if getattr(self, "h", None):
            h, self.h = self.h, None
            lib().mk_sync_status(h)
            lib().mk_destroy(h)

    def __del__(self, _finalizing=sys.is_finalizing):
        # at interpreter shutdown the exit hook has already closed the
        # handle; a finalizer that runs later (module globals may be gone,
        # hence the bound default) must not call into HIP
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
