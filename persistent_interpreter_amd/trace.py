"""Decode the megakernel's per-instruction trace (MK_FLAG_TRACE).

The library records, for every queued instruction of every workgroup, four
64-bit words: the opcode/layer/unit, the time its first waits were satisfied
(sync wave), the time compute wave 0 started it, and the time the last compute
wave finished it (100 MHz wall clock).  This module turns a raw buffer into
records, a per-(layer, instruction) summary and Perfetto/Chrome trace JSON.
"""
from __future__ import annotations

import json
from typing import Dict, List

import numpy as np

OPS = {1: "qkv", 2: "attn", 3: "attn_red", 4: "o_proj", 5: "ffn_gate_up",
       6: "ffn_down", 7: "lm_head"}
TICK_US = 0.01  # 100 MHz


def decode(raw: np.ndarray) -> np.ndarray:
    """Raw uint64 buffer -> structured records (cu, idx, op, layer, unit,
    t_wait, t_start, t_done) in microseconds from the earliest event."""
    raw = np.asarray(raw, dtype=np.uint64)
    ncu, stride = int(raw[0]), int(raw[1])
    rec = raw[4:4 + ncu * stride * 4].reshape(ncu, stride, 4)
    out = []
    for cu in range(ncu):
        for i in range(stride):
            w0, tw, ts, td = (int(x) for x in rec[cu, i])
            if w0 == 0 or tw == 0 or td == 0:
                continue
            out.append((cu, i, w0 & 0xFF, (w0 >> 8) & 0xFFFF, w0 >> 24, tw, ts, td))
    dt = np.dtype([("cu", "i4"), ("idx", "i4"), ("op", "i4"), ("layer", "i4"),
                   ("unit", "i4"), ("t_wait", "f8"), ("t_start", "f8"), ("t_done", "f8")])
    a = np.array(out, dtype=dt)
    if len(a):
        t0 = min(a["t_wait"].min(), a["t_start"].min())
        for f in ("t_wait", "t_start", "t_done"):
            a[f] = (a[f] - t0) * TICK_US
    return a


def summary(a: np.ndarray) -> List[Dict]:
    """Per (layer, op): earliest wait-satisfied, median and latest finish
    across workgroups, in microseconds."""
    rows = []
    for (layer, op) in sorted(set(zip(a["layer"], a["op"]))):
        m = (a["layer"] == layer) & (a["op"] == op)
        r = a[m]
        rows.append({"layer": int(layer), "op": OPS.get(int(op), str(op)),
                     "units": int(m.sum()),
                     "first_ready": float(r["t_wait"].min()),
                     "last_ready": float(r["t_wait"].max()),
                     "median_done": float(np.median(r["t_done"])),
                     "last_done": float(r["t_done"].max()),
                     "busy_med": float(np.median(r["t_done"] - r["t_start"]))})
    return rows


def perfetto(a: np.ndarray, path: str) -> None:
    """Chrome/Perfetto trace: one track per workgroup."""
    ev = []
    for r in a:
        ev.append({"name": f"L{r['layer']} {OPS.get(int(r['op']), r['op'])}",
                   "ph": "X", "pid": 0, "tid": int(r["cu"]),
                   "ts": float(r["t_start"]), "dur": float(r["t_done"] - r["t_start"]),
                   "args": {"unit": int(r["unit"]), "ready": float(r["t_wait"])}})
    with open(path, "w") as f:
        json.dump({"traceEvents": ev}, f)
