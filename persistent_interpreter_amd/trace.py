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


def _nanmed(x: np.ndarray) -> float:
    x = x[~np.isnan(x)]
    return float(np.median(x)) if len(x) else float("nan")


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
                     "xprod_med": _nanmed(r["t_xready"] - r["t_wait"]),
                     "epi_med": _nanmed(r["t_done"] - r["t_epi"])})
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


def main(argv=None) -> int:
    """Run traced greedy steps of a synthetic workload on the GPU and print
    the last step's per-(layer, instruction) summary and the per-layer
    critical path:

        python -m persistent_interpreter_amd.trace WORKLOAD [STEPS] [--kv-splits N]
                                                   [--steps-per-launch N]

With --steps-per-launch N each launch runs N chained greedy steps
(mk_decode_steps_greedy) and the trace holds the last launch's last step.

    Columns (microseconds from the step's first event): first/last time a
    unit's waits were satisfied, median/last completion, and medians of the
    unit's busy time (compute start to done), of the first activation
    piece's production and of the epilogue."""
    import argparse
    import ctypes

    from . import binding as B, harness, synth
    ap = argparse.ArgumentParser(prog="python -m persistent_interpreter_amd.trace")
    ap.add_argument("workload")
    ap.add_argument("steps", nargs="?", type=int, default=3)
    ap.add_argument("--kv-splits", type=int, default=0)
    ap.add_argument("--steps-per-launch", type=int, default=1)
    args = ap.parse_args(argv)
    spl = max(1, args.steps_per_launch)
    import torch
    mc = synth.CONFIGS[args.workload]
    mc = mc.replace(steps=max(mc.steps, args.steps * spl))
    W = synth.make_weights(mc, threads=16)
    kv = synth.make_kv_cache(mc, filled=mc.prior) if mc.batch == 1 else synth.make_kv_cache(mc)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)
    s = harness.Session(mc, W, kv, batch=mc.batch, flags=B.MK_FLAG_TRACE, kv_splits=args.kv_splits)
    s.set_inputs(tok, pos)
    lg = torch.empty(spl, mc.batch, mc.vocab, dtype=torch.float32, device="cuda")
    for _ in range(args.steps):
        if spl == 1:
            rc = s.step_greedy()
        else:
            rc = s.mk.decode_steps_greedy(mc.batch, spl, s.tokens, s.positions, s.kv, lg,
                                          s.tokens, s.positions)
        if rc != 0:
            raise RuntimeError(f"decode launch failed: {rc}")
    torch.cuda.synchronize()
    if s.mk.sync_status() != 0:
        raise RuntimeError("device error")
    ptr, nb = s.mk.buffer(B.MK_BUF_TRACE)
    raw = np.empty(nb // 8, np.uint64)
    hip = ctypes.CDLL("libamdhip64.so")
    if hip.hipMemcpy(ctypes.c_void_p(raw.ctypes.data), ctypes.c_void_p(ptr), ctypes.c_size_t(nb), 2) != 0:
        raise RuntimeError("hipMemcpy failed")
    s.close()
    a = decode(raw)
    span = float(np.nanmax(a["t_done"]) - np.nanmin(a["t_begin"]))
    what = "steps" if spl == 1 else f"launches of {spl} steps (the last step)"
    print(f"{args.workload}: last of {args.steps} traced {what}, span {span:.1f} us, {len(a)} records")
    print(f"{'L':>3} {'op':>12} {'units':>5} {'1st_rdy':>8} {'last_rdy':>8} {'med_done':>8} "
          f"{'last_done':>9} {'busy':>7} {'xprod':>6} {'epi':>6}")
    for r in summary(a):
        print(f"{r['layer']:>3} {r['op']:>12} {r['units']:>5} {r['first_ready']:8.1f} {r['last_ready']:8.1f} "
              f"{r['median_done']:8.1f} {r['last_done']:9.1f} {r['busy_med']:7.2f} {r['xprod_med']:6.2f} "
              f"{r['epi_med']:6.2f}")
    spans = []
    for layer in range(mc.n_layers):
        m = a["layer"] == layer
        q = m & (a["op"] == 1)
        spans.append(float(np.nanmax(a["t_done"][m]) - np.nanmin(a["t_wait"][q])))
    print(f"per-layer span (first QKV wait to last unit done), us: median {np.median(spans):.1f} "
          f"min {np.min(spans):.1f} max {np.max(spans):.1f}")
    return 0


if __name__ == "__main__":
    import sys
    sys.exit(main())
