#!/usr/bin/env python3
"""Decode benchmark of the persistent megakernel on one MI355X.

Workload: the Llama-1B-shaped decoder (16 layers, hidden 2048, 32/8 heads,
head_dim 64, SwiGLU 8192, vocab 128256, tied embeddings, RoPE theta 5e5) at
batch 1 with 512 prior KV positions, greedy decoding.  Weights and the KV
cache are seeded synthetic bf16 tensors (persistent_interpreter_amd.synth).

A step is the whole forward pass and the greedy next token and position,
computed by the persistent kernel, which writes them over its own token and
position buffers, so the timed steps chain on the device with no other
kernel or host round trip in between: one ``mk_decode_step_greedy`` launch
per step, or (``--steps-per-launch N``, the batch-8 default N = 8) one
``mk_decode_steps_greedy`` launch per N chained steps.  ``value``
is tokens/s over the K timed steps
(inputs resident in HBM).  ``roofline`` prices the megakernel against
MI355X's 8 TB/s: algorithmic bytes per launch (every weight byte once, the
embedding row, K and V of slots 0..p) over its average duration measured
with HIP events on the launch stream.  ``stream_read`` is the chip's
achievable streaming-read rate (``mk_stream_read`` over 2 GiB), the
practical ceiling of a step that reads every weight once, and the step's
share of it.  ``cpu_baseline`` times the CPU oracle
on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 32] [--warmup 3] [--workload llama1b]

``--workload llama1b_b8`` times the same shape at batch 8 (positions seeded
per sequence in [1024, 4096]); a step there is one launch of the batched
kernel, whose projections run on the matrix cores (bf16 hi + lo activation
splits), and ``roofline`` prices the whole step's algorithmic bytes (every
weight once, each sequence's K/V) over the step's duration; ``mfma_util``
gives the useful projection FLOP (2 x batch x weights) and the FLOP the
MFMA instructions issue (16 A rows: hi and lo of up to 8 sequences, tiles
padded to 16 weight rows) over the bf16 dense peak times the step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "decode tokens/s at batch 1 (Llama-1B shape) + % of peak HBM GB/s"
H100_STEP_S = 1.0e-3   # the pages' ~1 ms Llama-1B batch-1 forward on H100
# attention splits per (sequence, KV head) of each workload (0: the planner's
# choice)
DEFAULT_SPLITS = {}
# greedy steps per launch of each workload (measured: several steps per
# launch save about 70 us a step at batch 8 and cost about 14 us at batch 1,
# where the step hand-over inside the launch is slower than a new launch)
DEFAULT_SPL = {"llama1b_b8": 8}


def overhead(t_real: float, t_min: float) -> float:
    """Share of a step not explained by moving its bytes at peak bandwidth:
    (t_real - t_min) / t_real (chapter "Quand ne pas le faire", section 9.1)."""
    return (t_real - t_min) / t_real


def recovered(t_before: float, t_after: float, t_min: float) -> float:
    """Fraction of the removable time (t - t_min) a faster implementation
    recovered; the reading behind the section's MPK figure."""
    return (t_before - t_after) / (t_before - t_min)


def overhead_drop(bw_frac_before: float, bw_frac_after: float) -> float:
    """Relative drop of the overhead fraction when the share of peak
    bandwidth rises (t_min / t_real is that share); the reading behind the
    section's Hazy Research figure."""
    o0, o1 = 1.0 - bw_frac_before, 1.0 - bw_frac_after
    return (o0 - o1) / o0


def algorithmic_bytes(mc, positions) -> int:
    """Bytes a decode step must read: every weight tensor once, one
    embedding row per sequence, and K and V of slots 0..p of every layer."""
    b = mc.weight_bytes() + 2 * mc.hidden * len(positions)
    for p in positions:
        b += 2 * 2 * mc.n_layers * mc.n_kv_heads * mc.head_dim * (int(p) + 1)
    return b


def source_digest() -> str:
    """sha256 prefix over the kernel library's sources; a stored traffic
    figure is reported only for the source it was measured on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "persistent_interpreter_amd", "csrc", "*"))) + \
            [os.path.join(ROOT, "include", "mk.h")]:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_stem(workload: str) -> str:
    """Name of a workload's files under profiles/ (shape and batch)."""
    import re
    return workload if re.search(r"_b\d+$", workload) else workload + "_b1"


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this workload (copy-calibrated), or None when that summary is
    missing or was measured on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"mk_interp_{profile_stem(workload)}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    digest, val = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("Kernel source digest:"):
                digest = line.split(":", 1)[1].strip()
            elif line.startswith("traffic_bytes_per_launch:"):
                val = int(line.split(":", 1)[1].strip())
    return val if digest == source_digest() and val else None


def host_info() -> dict:
    """CPU model and RAM of the host the oracle runs on."""
    model, ram = "unknown", None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    ram = round(int(line.split()[1]) / 2**20, 1)
                    break
    except OSError:
        pass
    return {"cpu_model": model, "ram_gib": ram}


def cpu_baseline(mc, W, kv0, tok, pos, fed, gpu_logits, min_s=10.0, budget_s=30.0):
    """Time the CPU oracle on the same greedy run (teacher forced on the
    GPU's tokens) and compare its logits with the GPU's on the first pass.
    The run is repeated from the same starting cache until at least min_s
    seconds of oracle steps are timed (stopping at budget_s), so that the
    rate rests on seconds of CPU work even where the oracle is fast."""
    import oracle as O
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    Wf = O.upcast_weights(W)            # one-time decode of bf16 weights
    times, worst, match, compared, passes = [], 0.0, 0, 0, 0
    t_all = time.perf_counter()
    done = False
    while not done:
        kv = kv0.copy()
        for i in range(len(fed)):
            t0 = time.perf_counter()
            ref = O.decode_step(mc, Wf, fed[i], pos + i, kv)
            times.append(time.perf_counter() - t0)
            if passes == 0:
                worst = max(worst, float(np.abs(ref - gpu_logits[i]).max()))
                match += int(np.array_equal(np.argmax(ref, -1), np.argmax(gpu_logits[i], -1)))
                compared += 1
            if time.perf_counter() - t_all > budget_s and len(times) >= 2:
                done = True
                break
        passes += 1
        if time.perf_counter() - t_all >= min_s:
            done = True
    n = len(times)
    med = float(np.median(times))
    return ({"value": round(len(tok) / med, 3), "unit": "tokens/s", "cores": threads,
             "kind": "oracle", **host_info(),
             "sample": f"{n} decode steps ({passes} pass(es) over the {len(fed)} greedy steps of "
                       f"the same workload, {sum(times):.1f} s of oracle steps; numpy fp32 "
                       f"oracle, weights decoded to fp32 once beforehand), median "
                       f"{med * 1e3:.1f} ms/step"},
            {"max_abs_dlogit": worst, "greedy_match": f"{match}/{compared}"})


def mfma_util(mc, t_step: float) -> dict:
    """MFMA utilisation of a batched step: useful projection FLOP
    (2 x batch x projection weights) and the FLOP the 16x16x32 MFMAs issue
    (16 A rows, units' rows padded to 16-row tiles, K padded to 256), each
    over the dense bf16 peak times the step time."""
    from persistent_interpreter_amd import binding as B
    params = (mc.weight_bytes() // 2) - mc.hidden * (2 * mc.n_layers + 1)  # minus norm weights
    useful = 2.0 * mc.batch * params
    cfg = B.make_config(mc, max_batch=mc.batch)
    rc, rep = B.plan_check(cfg, mc.batch, 256)
    issued = 2.0 * 16 * rep.mfma_cols_k if rc == 0 else None
    peak = PEAK_BF16_TFLOPS * 1e12 * t_step
    return {"useful_tflop_per_step": round(useful / 1e12, 4),
            "useful_frac": round(useful / peak, 5),
            "issued_frac": round(issued / peak, 5) if issued else None,
            "peak_tflops": PEAK_BF16_TFLOPS}


STREAM_BYTES = 2 << 30


def stream_read_gbs(torch, stream, launches: int = 10) -> float:
    """The chip's achievable streaming-read rate (mk_stream_read over a
    2 GiB buffer, HIP events on the launch stream, mean of `launches`)."""
    import ctypes
    from persistent_interpreter_amd import binding as B
    L = B.lib()
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.empty(L.mk_stream_read_sink_words(), dtype=torch.int32, device="cuda")
    h = stream.cuda_stream

    def run():
        rc = L.mk_stream_read(ctypes.c_void_p(buf.data_ptr()), STREAM_BYTES,
                              ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(h))
        if rc != 0:
            raise RuntimeError(f"mk_stream_read failed: {rc}")

    run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(launches):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / launches
    del buf, sink
    return STREAM_BYTES / t / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
    ap.add_argument("--kv-splits", type=int, default=-1,
                    help="attention splits per (sequence, KV head); -1: the workload's default")
    ap.add_argument("--steps-per-launch", type=int, default=0,
                    help="greedy steps per launch (mk_decode_steps_greedy); must divide --steps; "
                         "0: the workload's default")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (for "
                         "scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path "
              "(batched workloads would shard as independent replicas, one per "
              "GPU, with no exchange; batch 1 would need tensor parallelism)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}))
        return

    from persistent_interpreter_amd import harness, synth
    mc = synth.CONFIGS[args.workload]
    K, Wu, spl = args.steps, args.warmup, args.steps_per_launch
    if spl == 0:
        spl = DEFAULT_SPL.get(args.workload, 1)
        while K % spl:
            spl //= 2
    if spl < 1 or K % spl:
        print("--steps-per-launch must be positive and divide --steps", file=sys.stderr)
        sys.exit(2)
    mc = mc.replace(steps=max(K, 32))
    W = synth.make_weights(mc, threads=16)
    kv0 = synth.make_kv_cache(mc, filled=mc.prior)
    tok, pos = synth.make_tokens(mc), synth.make_positions(mc)

    splits = DEFAULT_SPLITS.get(args.workload, 0) if args.kv_splits < 0 else args.kv_splits
    sess = harness.Session(mc, W, kv0.copy(), batch=mc.batch, kv_splits=splits)
    # untimed greedy pass whose logits the oracle checks
    n_check = min(K, 32)
    fed, gpu_logits = harness.greedy_run(sess, tok, pos, n_check)

    # warmup, then K timed greedy steps from the same start
    stream = torch.cuda.current_stream()
    sess.set_inputs(tok, pos)
    for _ in range(Wu):
        sess.step_checked()
    n_launch = K // spl
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_launch)]
    lg_multi = torch.empty(spl, mc.batch, mc.vocab, dtype=torch.float32, device="cuda") \
        if spl > 1 else None
    sess.set_inputs(tok, pos)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # K <= mc.steps: the cache has a slot for every timed step
    for i in range(n_launch):
        ev[i][0].record(stream)
        if spl == 1:
            rc = sess.step_greedy()
        else:
            rc = sess.mk.decode_steps_greedy(mc.batch, spl, sess.tokens, sess.positions, sess.kv,
                                             lg_multi, sess.tokens, sess.positions)
        ev[i][1].record(stream)
        if rc != 0:
            raise RuntimeError(f"decode launch failed: {rc}")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = sess.mk.sync_status()
    if st != 0:
        raise RuntimeError(f"device error {st}")
    # the device-chained run must feed the same tokens as the checked run
    # (the kernel is deterministic: same schedule, same reduction order)
    if K <= n_check:
        end_tok = sess.tokens.cpu().numpy()
        want = np.argmax(gpu_logits[K - 1], axis=-1)
        if not np.array_equal(end_tok, want):
            raise RuntimeError(f"in-kernel greedy chain diverged: {end_tok} != {want}")
    kern = np.array([a.elapsed_time(b) * 1e-3 for a, b in ev]) / spl   # seconds per step
    # the kernel instantiation the plan runs, as rocprofv3 names it
    from persistent_interpreter_amd import binding as Bnd
    rc_p, rep_p = Bnd.plan_check(Bnd.make_config(mc, max_batch=mc.batch, kv_splits=splits), mc.batch, 256)
    kernel_name = ("mk::mk_interp" + ("_b" if mc.batch > 1 else "") +
                   (("n" if mc.batch > 1 else "_n") if spl > 1 else "") +
                   ("<true>" if rc_p == 0 and rep_p.paged_kv else "<false>"))

    stream_gbs = stream_read_gbs(torch, stream)

    positions = [np.asarray(pos) + i for i in range(K)]
    bytes_per = float(np.mean([algorithmic_bytes(mc, p) for p in positions]))
    t_kern = float(np.mean(kern))
    achieved = bytes_per / t_kern / 1e9
    tok_s = mc.batch * K / wall
    prior = mc.prior if mc.batch == 1 else \
        f"{int(np.min(pos))}-{int(np.max(pos))} (seeded, U[{mc.pos_lo}, {mc.pos_hi}])"
    metric = METRIC if args.workload == "llama1b" else \
        f"decode tokens/s at batch {mc.batch} ({mc.name} shape) + % of peak HBM GB/s"
    out = {
        "metric": metric, "value": round(tok_s, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wu,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tok_s / (1.0 / H100_STEP_S), 4) if args.workload == "llama1b" else None,
        "baseline_ref": ("context only, not the target: the pages' ~1 ms Llama-1B batch-1 "
                         "forward on H100 (other hardware); the measured baseline is "
                         "cpu_baseline (the oracle), its ratio is vs_oracle")
                        if args.workload == "llama1b" else None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{mc.name}: {mc.n_layers} layers, hidden {mc.hidden}, "
                               f"{mc.n_q_heads}/{mc.n_kv_heads} heads x {mc.head_dim}, "
                               f"FFN {mc.ffn_dim}, vocab {mc.vocab}, batch {mc.batch}, "
                               f"{prior} prior KV positions, greedy (in-kernel argmax)",
                   "batch": mc.batch, "prior_positions": prior, "accumulate": "fp32",
                   "kv_splits": sess.mk.plan_splits(mc.batch),
                   "parallelism": "1 GPU, 1 persistent launch per step" if spl == 1 else
                                  f"1 GPU, 1 persistent launch per {spl} steps"},
        "kernel_us": {"mean": round(t_kern * 1e6, 2),
                      "median": round(float(np.median(kern)) * 1e6, 2),
                      "p10": round(float(np.percentile(kern, 10)) * 1e6, 2),
                      "p90": round(float(np.percentile(kern, 90)) * 1e6, 2)},
        "hbm_pct_of_peak": round(100 * achieved / PEAK_HBM_GBS, 2),
        "stream_read": {"gbs": round(stream_gbs, 1), "bytes": STREAM_BYTES,
                        "pct_of_peak": round(100 * stream_gbs / PEAK_HBM_GBS, 2),
                        "step_pct_of_stream": round(100 * achieved / stream_gbs, 2)},
        "overhead": round(overhead(t_kern, bytes_per / (PEAK_HBM_GBS * 1e9)), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": stored_traffic(args.workload),
                     "kernel": kernel_name,
                     "launches_per_step": 1.0 / spl,
                     "launch_us": round(t_kern * spl * 1e6, 2),
                     "bytes_per_step": int(bytes_per)},
    }
    if mc.batch > 1:
        out["mfma_util"] = mfma_util(mc, t_kern)
    if not args.no_cpu:
        cpu, parity = cpu_baseline(mc, W, kv0, tok, pos, fed, gpu_logits)
        out["cpu_baseline"] = cpu
        out["vs_oracle"] = round(tok_s / cpu["value"], 1)
        out["parity"] = parity
    sess.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
