#!/usr/bin/env python3
"""Benchmark of the multi-token Q8_0 mat-vec on one MI355X.

Workload: Q8_0 GEMV, 10240 rows x 2560 cols (27,852,800 packed weight bytes),
T = 1, 2, 3, 4 activation vectors.  One "step" is one call at each T (four
launches).  Weights are copied into a ring of identical buffers totalling
>= 1 GiB (more than 4x the 256 MB Infinity Cache) and the calls walk the ring,
so every call streams its weights from HBM.

Metric (as the pages count it): effective weight bandwidth = packed weight
bytes / time per call, 1 GB = 1e9 B, weight bytes counted once per call
whatever T is.  ``value`` = all weight bytes of the K timed steps / their wall
time on the launch stream (hipEvents), with every input already in HBM.

Prints ONE JSON line (rank 0).  ``--gpus`` above 1 is refused: this build runs
on one GPU.
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

from block_quantized_token_amd import _lib, inputs as I, ops  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "effective weight GB/s (and % of HBM peak) at T=1..4, Q8_0 2560x10240"
WORKLOAD = "c2a_q8_0_10240x2560"
ALSO = "c2b_q8_0_2560x6144"
RING_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ring_of(torch, W: np.ndarray, min_bytes: int = RING_BYTES):
    n = max(1, -(-min_bytes // W.nbytes))
    base = torch.from_numpy(W).cuda()
    return [base] + [base.clone() for _ in range(n - 1)]


def time_calls(torch, fmt, ring, x_dev, rows, T, calls, stream, y_dev):
    """Back-to-back calls over the ring between two events on ``stream``; returns ms."""
    entry = {0: _lib.qgemv_q8_0, 1: _lib.qgemv_q4_0, 2: _lib.qgemv_bf16}[fmt]
    cols = x_dev.shape[1]
    xp, yp, sp = x_dev.data_ptr(), y_dev.data_ptr(), stream.cuda_stream
    ptrs = [w.data_ptr() for w in ring]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(calls):
        st = entry(rows, cols, T, ptrs[i % len(ptrs)], xp, yp, sp)
        if st:
            _lib.check(st, "bench call")
    end.record(stream)
    return start, end


def cpu_baseline(case, budget_s: float):
    """The oracle, untuned, on the host cores: whole steps (T = 1..4) of the same
    workload repeated until about ``budget_s`` seconds have passed."""
    import oracle
    o = oracle.get()
    fmt, rows, cols, W, x = case["fmt"], case["rows"], case["cols"], case["W"], case["x"]
    nbytes = o.packed_bytes(fmt, rows, cols)
    steps, t0 = 0, time.perf_counter()
    while True:
        for T in (1, 2, 3, 4):
            o.gemv(fmt, rows, cols, W, x[:T])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=round(steps * 4 * nbytes / el / 1e9, 3), unit="GB/s", cores=o.num_threads(), kind="oracle",
                sample=f"{steps} full steps (T=1,2,3,4) of Q8_0 10240x2560 in {el:.1f} s",
                us_per_call=round(el / (steps * 4) * 1e6, 1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget; 0 skips the CPU leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the 2560x6144 detail timing")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} refused: this build measures one GPU only "
              "(the mat-vec shards by rows; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    _lib.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    case = I.dense_case(WORKLOAD)
    fmt, rows, cols = case["fmt"], case["rows"], case["cols"]
    nbytes = _lib.qg_packed_bytes(fmt, rows, cols)
    ring = ring_of(torch, case["W"])
    x_dev = torch.from_numpy(case["x"]).cuda()
    y_dev = torch.empty((4, rows), dtype=torch.float32, device="cuda")
    Ts = (1, 2, 3, 4)
    log(f"bench: {WORKLOAD} {nbytes} B/call, ring {len(ring)} copies, steps {args.steps}, warmup {args.warmup}")

    # warmup: every T, walking the ring
    for T in Ts:
        time_calls(torch, fmt, ring, x_dev[:T], rows, T, args.warmup, stream, y_dev)
    torch.cuda.synchronize()

    # timed region: exactly K steps (K calls at each T), grouped by T
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs = {T: time_calls(torch, fmt, ring, x_dev[:T], rows, T, args.steps, stream, y_dev) for T in Ts}
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms = {T: evs[T][0].elapsed_time(evs[T][1]) for T in Ts}
    total_ms = sum(ms.values())
    value = args.steps * len(Ts) * nbytes / (total_ms * 1e-3) / 1e9

    per_T = {}
    for T in Ts:
        us = ms[T] * 1e3 / args.steps
        per_T[str(T)] = dict(us_per_call=round(us, 3), gbs=round(nbytes / us / 1e3, 1),
                             pct_peak=round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1),
                             tile=ops.query_tile("q8_0", rows, cols, T))
    dom = max(Ts, key=lambda T: ms[T])
    dom_us = ms[dom] * 1e3 / args.steps
    achieved = nbytes / dom_us / 1e3

    detail = {}
    if not args.no_extra:
        c2 = I.dense_case(ALSO)
        r2 = ring_of(torch, c2["W"])
        x2 = torch.from_numpy(c2["x"]).cuda()
        y2 = torch.empty((4, c2["rows"]), dtype=torch.float32, device="cuda")
        nb2 = _lib.qg_packed_bytes(c2["fmt"], c2["rows"], c2["cols"])
        d2 = {}
        for T in Ts:
            time_calls(torch, c2["fmt"], r2, x2[:T], c2["rows"], T, 50, stream, y2)
            s, e = time_calls(torch, c2["fmt"], r2, x2[:T], c2["rows"], T, 1000, stream, y2)
            torch.cuda.synchronize()
            us = s.elapsed_time(e)
            d2[str(T)] = dict(us_per_call=round(us, 3), gbs=round(nb2 / us / 1e3, 1),
                              pct_peak=round(100 * nb2 / us / 1e3 / HBM_PEAK_GBS, 1))
        detail[ALSO] = d2
        del r2

    cpu = cpu_baseline(case, args.cpu_seconds) if args.cpu_seconds > 0 else None

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seed 0: fp16 scales |N(0,1)|*0.01, int8 codes U[-127,127], x N(0,1))",
        "config": {"workload": "Q8_0 GEMV 10240 rows x 2560 cols, T=1,2,3,4 (one call per T per step)",
                   "rows": rows, "cols": cols, "weight_bytes_per_call": nbytes, "ring_copies": len(ring),
                   "ring_bytes": nbytes * len(ring), "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "per_T": per_T,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": f"qgemv_dense_kernel<Q8_0, T={dom}>", "us_per_launch": round(dom_us, 3),
                     "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "detail": detail,
        "wall_s_timed_region": round(wall_s, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
