"""Decode the megakernel's per-instruction trace (MK_FLAG_TRACE).

The library records, for every queued instruction of every workgroup, eight
64-bit words: the opcode/layer/unit and six timestamps (100 MHz wall clock)
of the sync wave and the compute waves (see ``decode``).  This module turns a raw buffer into
records, a per-(layer, instruction) summary and Perfetto/Chrome trace JSON.
"""
from __future__ import annotations

import json
from typing import Dict, List

import numpy as np

OPS = {1: "qkv", 2: "attn", 3: "attn_red", 4: "o_proj", 5: "ffn_gate_up",
       6: "ffn_down", 7: "lm_head"}
TICK_US = 0.01  # 100 MHz


FIELDS = ("t_wait", "t_start", "t_done", "t_begin", "t_xready", "t_epi", "t_xlast")


def decode(raw: np.ndarray) -> np.ndarray:
    """Raw uint64 buffer -> structured records (cu, idx, op, layer, unit and
    the timestamps below) in microseconds from the earliest event.

    t_begin  sync wave started the instruction (before its counter waits)
    t_wait   its waits for the first activation piece were satisfied
    t_xready the first activation piece was published in LDS
    t_start  compute wave 0 passed the unit's gate
    t_epi    the last compute wave finished its pieces (epilogue starts)
    t_done   epilogue done, counters about to be signalled
    t_xlast  the last activation piece was published (= t_xready for one)"""
    raw = np.asarray(raw, dtype=np.uint64)
    ncu, stride = int(raw[0]), int(raw[1])
    words = int(raw[2]) or 4
    rec = raw[4:4 + ncu * stride * words].reshape(ncu, stride, words).astype(np.int64)
    out = []
    for cu in range(ncu):
        for i in range(stride):
            r = rec[cu, i]
            if r[0] == 0 or r[1] == 0 or r[3] == 0:
                continue
            ext = [r[4], r[5], r[6], r[7]] if words >= 8 else [r[1], r[1], r[3], r[1]]
            out.append((cu, i, r[0] & 0xFF, (r[0] >> 8) & 0xFFFF, r[0] >> 24, r[1], r[2], r[3], *ext))
    dt = np.dtype([("cu", "i4"), ("idx", "i4"), ("op", "i4"), ("layer", "i4"), ("unit", "i4"),
                   ("t_wait", "f8"), ("t_start", "f8"), ("t_done", "f8"),
                   ("t_begin", "f8"), ("t_xready", "f8"), ("t_epi", "f8"), ("t_xlast", "f8")])
    a = np.array(out, dtype=dt)
    if len(a):
        valid = [a[f][a[f] > 0] for f in FIELDS]
        t0 = min(v.min() for v in valid if len(v))
        for f in FIELDS:
            a[f] = np.where(a[f] > 0, (a[f] - t0) * TICK_US, np.nan)
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
                     "busy_med": float(np.median(r["t_done"] - r["t_start"])),
                     "xprod_med": float(np.nanmedian(r["t_xready"] - r["t_wait"])),
                     "epi_med": float(np.nanmedian(r["t_done"] - r["t_epi"]))})
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
