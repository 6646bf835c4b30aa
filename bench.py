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

Prints ONE JSON line (rank 0).  ``--gpus`` above 1 is refused: the benchmark runs
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
KERNEL_SRC = os.path.join(ROOT, "block_quantized_token_amd", "csrc", "qgemv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemv_q8_0_10240x2560_hbm_traffic.txt")
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
    """Back-to-back calls over the ring between two events on ``stream``; returns the (start, end) events."""
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


def kernel_name(tile, T):
    """Device symbol of the kernel a call with ``tile`` launches (Q8_0)."""
    if tile["kind"] == 9:
        return f"qgemv_mxp_kernel<0, {T}>"
    if tile["kind"] == 11:
        return f"qgemv_mx_kernel<0, {T}, 1, 2>"
    if tile["kind"] == 8:
        return f"qgemv_mx_kernel<0, {T}, {2 if tile['depth'] == 2 else 1}, 1>"
    if tile["kind"] == 7:
        return f"qgemv_half_kernel<0, {T}, {tile['depth']}>"
    if tile["kind"] in (2, 3):
        return f"qgemv_dma_kernel<0, {T}, {2 * tile['rows_per_batch']}, {tile['depth']}, {str(tile['kind'] == 3).lower()}>"
    if tile["kind"] == 1 and tile["mfma"] == 2:
        return f"qgemv_mfma_persist_kernel<{T}>"
    if tile["kind"] == 1 and tile["mfma"]:
        return f"qgemv_mfma_q8_kernel<{T}>"
    if tile["kind"] == 4:
        return f"qgemv_units_kernel<0, {T}, {tile['depth']}>"
    if tile["kind"] == 1:
        return f"qgemv_stream_kernel<0, {T}, {2 * tile['rows_per_batch']}>"
    one_shot = str(tile["rows_per_wg"] == 2 * tile["rows_per_batch"]).lower()
    return f"qgemv_dense_kernel<0, {T}, {tile['rows_per_batch']}, {one_shot}>"


def source_digest():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of ``kernel`` from the committed PMC summary, or None
    when there is none or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields, rows = {}, {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line.startswith("kernel_source_sha256:"):
            fields["digest"] = line.split(":", 1)[1].strip()
        elif line.startswith("| ") and "|" in line[2:]:
            cells = [c.strip() for c in line.strip("|").split("|")]
            if len(cells) >= 5 and cells[0] != "kernel" and not cells[0].startswith("-"):
                rows[cells[0]] = cells
    if fields.get("digest") != source_digest() or kernel not in rows:
        return None
    return int(float(rows[kernel][4]))


def summarize_pmc(fetch_dir, write_dir, nbytes, alg_bytes=None):
    """Per-kernel HBM traffic from two rocprofv3 --pmc runs of this script
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the calibration copy (nbytes read, nbytes written), set
    beside ``alg_bytes`` algorithmic bytes per launch (default nbytes)."""
    alg_bytes = alg_bytes or nbytes
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            sys.exit(f"no counter_collection.csv under {d}")
        acc = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].replace("void ", "").replace("qg::(anonymous namespace)::", "")
                name = name.split("(")[0]
                acc.setdefault(name, {}).setdefault(r["Dispatch_Id"], 0.0)
                acc[name][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sorted(v.values())[len(v) // 2] for k, v in acc.items()}  # median over dispatches

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    cal = [k for k in fetch if "MulFunctor" in k]  # torch.mul(src, 1.0, out=dst): reads and writes nbytes
    if not cal:
        sys.exit("calibration copy kernel not found in the FETCH_SIZE run")
    cal = cal[0]
    f_scale = nbytes / (fetch[cal] * 1024.0)
    w_scale = nbytes / (write[cal] * 1024.0)
    print(f"kernel_source_sha256: {source_digest()}")
    print(f"calibration: {cal} moves {nbytes} B each way; FETCH_SIZE reads {fetch[cal]:.1f} KiB "
          f"(scale {f_scale:.4f}), WRITE_SIZE reads {write[cal]:.1f} KiB (scale {w_scale:.4f})")
    print(f"algorithmic bytes per launch: {alg_bytes} weight bytes (+ x and y)")
    print()
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read B | scaled read + write B | vs algorithmic |")
    print("|---|---|---|---|---|---|")
    for k in sorted(fetch):
        if k == cal or not k.startswith("qgemv"):
            continue
        rb = fetch[k] * 1024.0 * f_scale
        wb = write.get(k, 0.0) * 1024.0 * w_scale
        print(f"| {k} | {fetch[k]:.1f} | {write.get(k, 0.0):.1f} | {rb:.0f} | {rb + wb:.0f} | {(rb + wb) / alg_bytes:.3f} |")


def time_entry(torch, stream, launch, calls):
    """µs per call of ``launch(i)``: the median of 3 runs of ``calls`` back-to-back
    calls each (after 20 warm-up calls)."""
    for i in range(20):
        launch(i)
    runs = []
    for _ in range(3):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for i in range(calls):
            launch(i)
        e.record(stream)
        torch.cuda.synchronize()
        runs.append(s.elapsed_time(e) * 1e3 / calls)
    return sorted(runs)[1]


def other_workloads(torch, stream):
    """The other shapes the pages time, T = 1..4, for the record (not part of
    ``value``).  Timing does not depend on the weight values, so each ring copy is
    random bytes drawn on the device; every call streams from HBM (ring >= 1 GiB)."""
    out = {}
    sp = stream.cuda_stream
    for name in ("c1_q8_0_2560x2560", "c2b_q8_0_2560x6144", "c3_q4_0_8192x2560", "c3_bf16_8192x2560",
                 "c4_q8_0_248320x5120"):
        fmt, rows, cols, _ = I.CONFIGS[name]
        nb = _lib.qg_packed_bytes(fmt, rows, cols)
        ring = [torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda")
                for _ in range(max(1, -(-RING_BYTES // nb)))]
        x = torch.randn(4, cols, device="cuda")
        y = torch.empty(4, rows, device="cuda")
        entry = {0: _lib.qgemv_q8_0, 1: _lib.qgemv_q4_0, 2: _lib.qgemv_bf16}[fmt]
        calls = max(50, min(2000, int(4e9 / nb)))
        res = {}
        for T in (1, 2, 3, 4):
            def launch(i, T=T):
                st = entry(rows, cols, T, ring[i % len(ring)].data_ptr(), x.data_ptr(), y.data_ptr(), sp)
                if st:
                    _lib.check(st, name)
            us = time_entry(torch, stream, launch, calls)
            res[str(T)] = dict(us_per_call=round(us, 3), gbs=round(nb / us / 1e3, 1),
                               pct_peak=round(100 * nb / us / 1e3 / HBM_PEAK_GBS, 1),
                               tile=ops.query_tile(I.FMT_NAMES[fmt], rows, cols, T))
        if name == "c4_q8_0_248320x5120":  # the fused LM-head argmax (y never written)
            idx = torch.empty(4, dtype=torch.int32, device="cuda")
            val = torch.empty(4, device="cuda")
            work = torch.empty(4, dtype=torch.int64, device="cuda")
            am = {}
            for T in (1, 2, 3, 4):
                def launch(i, T=T):
                    st = _lib.qgemv_argmax(fmt, rows, cols, T, ring[i % len(ring)].data_ptr(), x.data_ptr(),
                                           work.data_ptr(), idx.data_ptr(), val.data_ptr(), sp)
                    if st:
                        _lib.check(st, "argmax")
                us = time_entry(torch, stream, launch, calls)
                am[str(T)] = dict(us_per_call=round(us, 3), gbs=round(nb / us / 1e3, 1),
                                  pct_peak=round(100 * nb / us / 1e3 / HBM_PEAK_GBS, 1))
            out["c4_argmax_fused"] = dict(weight_bytes_per_call=nb, calls=calls, per_T=am)
            # a draft vocabulary: 32,768 distinct rows of the head, sorted, read through the row subset
            # (7 disjoint vocabularies in turn, 1.25 GB together, so each call's rows come from HBM)
            nsel = 32768
            perm = torch.randperm(rows, device="cuda")
            idsets = [torch.sort(perm[j * nsel:(j + 1) * nsel].to(torch.int32)).values for j in range(rows // nsel)]
            ys = torch.empty(4, nsel, device="cuda")
            sub = nsel * (nb // rows)
            rs = {}
            for T in (1, 2, 3, 4):
                def launch(i, T=T):
                    st = _lib.qgemv_rows(fmt, rows, cols, nsel, idsets[i % len(idsets)].data_ptr(), T,
                                         ring[0].data_ptr(), x.data_ptr(), ys.data_ptr(), sp)
                    if st:
                        _lib.check(st, "rows")
                us = time_entry(torch, stream, launch, max(200, calls))
                rs[str(T)] = dict(us_per_call=round(us, 3), bytes_read=sub, gbs=round(sub / us / 1e3, 1),
                                  pct_peak=round(100 * sub / us / 1e3 / HBM_PEAK_GBS, 1))
            out["c4_rows_32768"] = dict(n_sel=nsel, vocabularies=len(idsets), per_T=rs)
        out[name] = dict(weight_bytes_per_call=nb, calls=calls, ring_copies=len(ring), per_T=res)
        del ring
    # grouped experts: 256 Q4_0 experts of 512 x 2560; each token picks 10 distinct
    # experts, none shared; bytes per call = the distinct experts' bytes
    g = I.GROUPED["c5_q4_0_experts"]
    E, rows, cols, topk = g["n_experts"], g["rows"], g["cols"], g["topk"]
    table = _lib.qg_packed_bytes(g["fmt"], E * rows, cols)
    ring = [torch.randint(0, 256, (table,), dtype=torch.uint8, device="cuda")
            for _ in range(max(1, -(-RING_BYTES // table)))]
    ids_all = torch.from_numpy(I.expert_ids(I.rng_for(0), E, 4, topk)).cuda()
    x = torch.randn(4, cols, device="cuda")
    y = torch.empty(4, topk, rows, device="cuda")
    res = {}
    for T in (1, 2, 3, 4):
        ids = ids_all[:T].contiguous()
        nb = T * topk * table // E  # distinct experts read
        def launch(i, T=T, ids=ids):
            st = _lib.qgemv_grouped_experts(g["fmt"], E, rows, cols, T, topk, ids.data_ptr(),
                                            ring[i % len(ring)].data_ptr(), x.data_ptr(), y.data_ptr(), sp)
            if st:
                _lib.check(st, "grouped")
        us = time_entry(torch, stream, launch, 1000)
        res[str(T)] = dict(us_per_call=round(us, 3), bytes_read=nb, gbs=round(nb / us / 1e3, 1),
                           pct_peak=round(100 * nb / us / 1e3 / HBM_PEAK_GBS, 1))
    out["c5_q4_0_experts"] = dict(table_bytes=table, ring_copies=len(ring), topk=topk, per_T=res)
    del ring
    # the routed-experts layer: gate+up (one launch, two tables) then down, at the
    # audit's expert overlap (share 0.65) and with none; bytes = distinct experts'
    # gate, up and down tables
    L = I.EXPERT_LAYER
    E, ff, emb, topk, lf = L["n_experts"], L["n_ff"], L["n_embd"], L["topk"], L["fmt"]
    tb = _lib.qg_packed_bytes(lf, E * ff, emb)  # one table (gate, up and down are the same size)
    copies = max(1, -(-RING_BYTES // (3 * tb)))
    tabs = [[torch.randint(0, 256, (tb,), dtype=torch.uint8, device="cuda") for _ in range(3)] for _ in range(copies)]
    x = torch.randn(4, emb, device="cuda")
    h = torch.randn(4, topk, ff, device="cuda")
    yg = torch.empty(4, topk, ff, device="cuda")
    yu = torch.empty_like(yg)
    yd = torch.empty(4, topk, emb, device="cuda")
    for share in ("0.65", "0"):
        res = {}
        for T in (1, 2, 3, 4):
            unique = I.UNIQUE_AT_SHARE_065[T] if share == "0.65" else topk * T
            ids = torch.from_numpy(I.expert_ids_shared(I.rng_for(T), E, T, topk, unique)).cuda()
            def gu(i, T=T, ids=ids):
                Wg, Wu, _ = tabs[i % copies]
                st = _lib.qgemv_experts_gate_up(lf, E, ff, emb, T, topk, ids.data_ptr(), Wg.data_ptr(), Wu.data_ptr(),
                                                x.data_ptr(), yg.data_ptr(), yu.data_ptr(), sp)
                if st:
                    _lib.check(st, "gate_up")
            def dn(i, T=T, ids=ids):
                st = _lib.qgemv_experts_down(lf, E, emb, ff, T, topk, ids.data_ptr(), tabs[i % copies][2].data_ptr(),
                                             h.data_ptr(), yd.data_ptr(), sp)
                if st:
                    _lib.check(st, "down")
            def layer(i):
                gu(i)
                dn(i)
            per = tb // E
            r = {}
            for label, fn, nbytes in (("gate_up", gu, 2 * unique * per), ("down", dn, unique * per),
                                      ("layer", layer, 3 * unique * per)):
                us = time_entry(torch, stream, fn, 1000)
                r[label] = dict(us_per_call=round(us, 3), bytes_read=nbytes, gbs=round(nbytes / us / 1e3, 1),
                                pct_peak=round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1))
            res[str(T)] = dict(distinct_experts=unique, **r)
        out[f"expert_layer_q4_0_share{share}"] = dict(table_bytes=tb, ring_copies=copies, per_T=res)
    del tabs
    # on-device quantizers: fp32 in, packed blocks out; bytes = fp32 read + packed written
    for label, fmt, method, rows, cols in (("quantize_q8_0_10240x2560", I.FMT_Q8_0, 0, 10240, 2560),
                                           ("quantize_q4_0_absmax_8192x2560", I.FMT_Q4_0, 0, 8192, 2560),
                                           ("quantize_q4_0_lloyd_8192x2560", I.FMT_Q4_0, 1, 8192, 2560)):
        sb = rows * cols * 4
        nb = _lib.qg_packed_bytes(fmt, rows, cols)
        srcs = [torch.randn(rows, cols, device="cuda") * 0.02 for _ in range(max(1, -(-RING_BYTES // sb)))]
        dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
        def launch(i, fmt=fmt, method=method, rows=rows, cols=cols):
            a = srcs[i % len(srcs)].data_ptr()
            st = (_lib.qg_quantize_q8_0(rows, cols, a, dst.data_ptr(), sp) if fmt == I.FMT_Q8_0 else
                  _lib.qg_quantize_q4_0(rows, cols, method, a, dst.data_ptr(), sp))
            if st:
                _lib.check(st, "quantize")
        us = time_entry(torch, stream, launch, 300)
        out[label] = dict(bytes_per_call=sb + nb, read=sb, written=nb, ring_copies=len(srcs), us_per_call=round(us, 3),
                          gbs=round((sb + nb) / us / 1e3, 1), pct_peak=round(100 * (sb + nb) / us / 1e3 / HBM_PEAK_GBS, 1))
        del srcs
    return out


def read_probe(torch, stream, nbytes):
    """Context for the roofline: the library's plain read kernel (qg_read_probe:
    coalesced 16-byte loads, nothing else) over ``nbytes`` streamed from HBM (a
    ring of >= 1 GiB, as the mat-vec's weights) and over one 1 GiB buffer; the
    fastest of a few workgroup limits for each."""
    sp = stream.cuda_stream
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ring = [torch.full((nbytes // 4,), 1, dtype=torch.int32, device="cuda") for _ in range(max(1, -(-RING_BYTES // nbytes)))]
    big = torch.full((RING_BYTES // 4,), 1, dtype=torch.int32, device="cuda")
    res = {"kernel": "read_probe_kernel (qg_read_probe)"}
    for label, bufs, size, calls in (("bench_size", ring, nbytes, 400), ("1gib", [big], RING_BYTES, 20)):
        best = None
        for groups in (512, 1024, 2048, 4096, 8192):
            def launch(i, bufs=bufs, size=size, groups=groups):
                st = _lib.qg_read_probe(bufs[i % len(bufs)].data_ptr(), size, groups, 0xFFFFFFFF, out.data_ptr(), sp)
                if st:
                    _lib.check(st, "read probe")
            us = time_entry(torch, stream, launch, calls)
            if best is None or us < best[0]:
                best = (us, groups)
        res[label] = dict(bytes=size, us_per_call=round(best[0], 3), gbs=round(size / best[0] / 1e3, 1),
                          pct_peak=round(100 * size / best[0] / 1e3 / HBM_PEAK_GBS, 1), max_groups=best[1])
    del ring, big
    return res


def host_info(torch):
    """What the numbers were measured on: host CPU, ROCm, torch and the GPU."""
    info = {"cpu_model": None, "logical_cpus": os.cpu_count()}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        info["rocm_version"] = open(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), ".info", "version")).read().strip()
    except OSError:
        info["rocm_version"] = None
    info["torch"] = torch.__version__
    info["hip_runtime"] = getattr(torch.version, "hip", None)
    props = torch.cuda.get_device_properties(0)
    info["gpu"] = props.name
    info["gpu_arch"] = getattr(props, "gcnArchName", None)
    info["compute_units"] = props.multi_processor_count
    return info


def _numeric_leaves(obj, path=""):
    if isinstance(obj, dict):
        for k, v in obj.items():
            yield from _numeric_leaves(v, f"{path}.{k}" if path else str(k))
    elif isinstance(obj, list):
        for i, v in enumerate(obj):
            yield from _numeric_leaves(v, f"{path}[{i}]")
    elif isinstance(obj, (int, float)) and not isinstance(obj, bool):
        yield path, obj


CLOCK_CMD = ["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"]


def under_profiler():
    """True when a rocprofv3 tool library is preloaded: its children (amd-smi is a
    Python script started through env) would inherit it, so no clock is sampled."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "")


def gpu_clocks():
    """One amd-smi sample of GPU 0's clocks and power (a child process; the values
    are what the tool reports, MHz and W), or the reason there is none."""
    import subprocess
    if under_profiler():
        return {"skipped": "under rocprofv3"}
    try:
        r = subprocess.run(CLOCK_CMD, capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError) as e:
        return {"error": f"amd-smi: {type(e).__name__}: {str(e)[:200]}"}
    return _parse_clocks(r.stdout)


def _parse_clocks(text):
    try:
        keep = clock_fields(json.loads(text))
    except ValueError as e:
        return {"error": f"amd-smi output: {str(e)[:200]}"}
    return keep if keep else {"raw": text[:400]}


def clocks_under_load(torch, batch, min_s):
    """Run ``batch()`` (a few calls of the workload) back to back for at least
    ``min_s`` seconds while one amd-smi sample is taken, so the sample shows the
    clocks the calls run at (an idle GPU drops to its idle clock within a fraction
    of a second); returns the sample."""
    import subprocess
    p = None
    if under_profiler():
        res = {"skipped": "under rocprofv3"}
    else:
        try:
            p = subprocess.Popen(CLOCK_CMD, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError as e:
            res = {"error": f"amd-smi: {type(e).__name__}: {str(e)[:200]}"}
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s or (p is not None and p.poll() is None):
        batch()
        torch.cuda.synchronize()
        if p is not None and time.perf_counter() - t0 > 30:
            p.kill()
    if p is not None:
        out, _ = p.communicate()
        res = _parse_clocks(out)
    return res


def clock_fields(data):
    """The gfx / memory clock and power values of an amd-smi metric JSON document."""
    keep = {}
    for path, v in _numeric_leaves(data):
        p = path.lower()
        if ("gfx" in p or "mem" in p or "power" in p) and (".clk." in p or "power" in p) and "value" in p:
            keep[path] = v
    return dict(list(keep.items())[:24])


def _median_call(fn, repeats):
    runs = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        fn()
        runs.append(time.perf_counter() - t0)
    runs.sort()
    return runs[len(runs) // 2]


def cpu_baseline(case, budget_s: float):
    """The oracle, untuned, on the host cores: whole steps (T = 1..4) of the same
    workload repeated until about ``budget_s`` seconds have passed; the value is
    their total rate, with the median of the step times beside it."""
    import oracle
    o = oracle.get()
    fmt, rows, cols, W, x = case["fmt"], case["rows"], case["cols"], case["W"], case["x"]
    nbytes = o.packed_bytes(fmt, rows, cols)
    steps, t0, step_s = 0, time.perf_counter(), []
    while True:
        ts = time.perf_counter()
        for T in (1, 2, 3, 4):
            o.gemv(fmt, rows, cols, W, x[:T])
        step_s.append(time.perf_counter() - ts)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s and steps >= 3:
            break
    step_s.sort()
    med = step_s[len(step_s) // 2]
    return dict(value=round(steps * 4 * nbytes / el / 1e9, 3), unit="GB/s", cores=o.num_threads(), kind="oracle",
                sample=f"{steps} full steps (T=1,2,3,4) of Q8_0 10240x2560 in {el:.1f} s",
                us_per_call=round(el / (steps * 4) * 1e6, 1),
                median_step_gbs=round(4 * nbytes / med / 1e9, 3), median_step_s=round(med, 4))


def cpu_baseline_per_workload():
    """The oracle on every other workload at full size, at T = 1..4: the median of 3
    runs (one for the 1.35 GB LM head) on all host threads; and on one thread for
    the dense configs C1-C3 at T = 1 and 4 (median of 3).  Seeded inputs of each
    workload's shape."""
    import oracle
    o = oracle.get()
    threads = o.num_threads()
    out = {}
    single = {}
    for name in ("c1_q8_0_2560x2560", "c2a_q8_0_10240x2560", "c2b_q8_0_2560x6144", "c3_q4_0_8192x2560",
                 "c3_bf16_8192x2560", "c4_q8_0_248320x5120"):
        c = I.dense_case(name)
        fmt, rows, cols, W, x = c["fmt"], c["rows"], c["cols"], c["W"], c["x"]
        nb = o.packed_bytes(fmt, rows, cols)
        reps = 1 if rows * cols > (1 << 28) else 3
        res = {}
        for T in (1, 2, 3, 4):
            s_ = _median_call(lambda T=T: o.gemv(fmt, rows, cols, W, x[:T]), reps)
            res[str(T)] = dict(us_per_call=round(s_ * 1e6, 1), gbs=round(nb / s_ / 1e9, 3))
        if name != "c2a_q8_0_10240x2560":
            out[name] = dict(sample=f"all {rows} rows, median of {reps}", threads=threads, per_T=res)
        if name != "c4_q8_0_248320x5120":
            o.set_num_threads(1)
            try:
                r1 = {}
                for T in (1, 4):
                    s_ = _median_call(lambda T=T: o.gemv(fmt, rows, cols, W, x[:T]), 3)
                    r1[str(T)] = dict(us_per_call=round(s_ * 1e6, 1), gbs=round(nb / s_ / 1e9, 4))
            finally:
                o.set_num_threads(threads)
            single[name] = r1
        del c, W
    g = I.grouped_case()
    res = {}
    for T in (1, 2, 3, 4):
        ids = g["ids"][:T]
        s_ = _median_call(lambda T=T, ids=ids: o.grouped(g["fmt"], g["n_experts"], g["rows"], g["cols"], ids, g["W"],
                                                          g["x"][:T]), 3)
        nb = T * g["topk"] * o.packed_bytes(g["fmt"], g["rows"], g["cols"])
        res[str(T)] = dict(us_per_call=round(s_ * 1e6, 1), gbs=round(nb / s_ / 1e9, 3))
    out["c5_q4_0_experts"] = dict(sample="every slot, median of 3", threads=threads, per_T=res)
    out["single_thread"] = dict(sample="all rows, T = 1 and 4, median of 3, one host thread", per_workload=single)
    return out


def _kernel_short(name):
    return name.replace("void ", "").replace("qg::(anonymous namespace)::", "").split("(")[0]


def summarize_trace(trace_dir, skip_first=0):
    """Per-kernel call count and duration from a rocprofv3 --kernel-trace --stats run;
    with ``skip_first`` the run's first that many dispatches of this library's kernels
    (by start time) are left out, so a pass that only brings the clocks up is not counted."""
    import csv
    import glob
    print(f"kernel_source_sha256: {source_digest()}")
    print()
    share = "share of this library's kernel time" if skip_first else "share of kernel time"
    print(f"| kernel | calls | average us | min us | max us | {share} |")
    print("|---|---|---|---|---|---|")
    if skip_first:
        files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
        if not files:
            sys.exit(f"no kernel_trace.csv under {trace_dir}")
        recs = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Start_Timestamp"]))
        recs = [r for r in recs if _kernel_short(r["Kernel_Name"]).startswith(("qgemv", "quantize"))][skip_first:]
        acc = {}
        for r in recs:
            acc.setdefault(_kernel_short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        total = sum(sum(v) for v in acc.values())
        for name, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            print(f"| {name} | {len(v)} | {sum(v) / len(v):.3f} | {min(v):.3f} | {max(v):.3f} | "
                  f"{100 * sum(v) / total:.2f}% |")
        return
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_stats.csv under {trace_dir}")
    for r in csv.DictReader(open(files[0])):
        name = _kernel_short(r["Name"])
        if not name.startswith(("qgemv", "quantize")):
            continue
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | {int(r['MinNs']) / 1e3:.3f} | "
              f"{int(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f}% |")


def summarize_counters(counter_dir):
    """Per-kernel medians over dispatches of every counter of a rocprofv3 --pmc run."""
    import csv
    import glob
    files = glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no counter_collection.csv under {counter_dir}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            name = _kernel_short(r["Kernel_Name"])
            if not name.startswith("qgemv"):
                continue
            d = acc.setdefault(name, {}).setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    print(f"kernel_source_sha256: {source_digest()}")
    counters = sorted({c for v in acc.values() for c in v})
    print()
    print("| kernel | " + " | ".join(counters) + " |")
    print("|---" * (len(counters) + 1) + "|")
    for k in sorted(acc):
        med = [sorted(acc[k][c].values())[len(acc[k][c]) // 2] if c in acc[k] else float("nan") for c in counters]
        print(f"| {k} | " + " | ".join(f"{m:.4g}" for m in med) + " |")


PROFILE_WORKLOADS = ("c1_q8_0_2560x2560", "c2a_q8_0_10240x2560", "c2b_q8_0_2560x6144", "c3_q4_0_8192x2560",
                     "c3_bf16_8192x2560", "c4_q8_0_248320x5120", "c4_argmax", "c5_q4_0_experts")


def profile_workload(torch, stream, name, calls, tiles, Ts=(1, 2, 3, 4)):
    """Untimed calls for rocprofv3 to trace or count: ``calls`` calls at each T in ``Ts``
    of one workload for each tile spec in ``tiles`` ("default" = the library's own
    tile; a spec outside what the library runs at some T is skipped there), walking a
    ring of device-random weights of >= 1 GiB so every call streams from HBM."""
    import os as _os
    sp = stream.cuda_stream
    if name == "c5_q4_0_experts":
        g = I.GROUPED[name]
        E, rows, cols, topk = g["n_experts"], g["rows"], g["cols"], g["topk"]
        nb = _lib.qg_packed_bytes(g["fmt"], E * rows, cols)
        ring = [torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda") for _ in range(max(1, -(-RING_BYTES // nb)))]
        ids_all = torch.from_numpy(I.expert_ids(I.rng_for(0), E, 4, topk)).cuda()
        x = torch.randn(4, cols, device="cuda")
        y = torch.empty(4, topk, rows, device="cuda")
        fmt_name = I.FMT_NAMES[g["fmt"]]

        def call(T, i):
            ids = ids_all[:T].contiguous()
            return _lib.qgemv_grouped_experts(g["fmt"], E, rows, cols, T, topk, ids.data_ptr(), ring[i % len(ring)].data_ptr(),
                                              x.data_ptr(), y.data_ptr(), sp)
    else:
        base = "c4_q8_0_248320x5120" if name == "c4_argmax" else name
        fmt, rows, cols, _ = I.CONFIGS[base]
        fmt_name = I.FMT_NAMES[fmt]
        nb = _lib.qg_packed_bytes(fmt, rows, cols)
        ring = [torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda") for _ in range(max(1, -(-RING_BYTES // nb)))]
        x = torch.randn(4, cols, device="cuda")
        y = torch.empty(4, rows, device="cuda")
        entry = {0: _lib.qgemv_q8_0, 1: _lib.qgemv_q4_0, 2: _lib.qgemv_bf16}[fmt]
        work = torch.empty(4, dtype=torch.int64, device="cuda")
        idx = torch.empty(4, dtype=torch.int32, device="cuda")
        val = torch.empty(4, device="cuda")

        def call(T, i):
            W = ring[i % len(ring)].data_ptr()
            if name == "c4_argmax":
                return _lib.qgemv_argmax(fmt, rows, cols, T, W, x.data_ptr(), work.data_ptr(), idx.data_ptr(),
                                         val.data_ptr(), sp)
            return entry(rows, cols, T, W, x.data_ptr(), y.data_ptr(), sp)
    for w in ring:  # first touch of fresh memory outside the traced calls
        torch.count_nonzero(w)
    torch.cuda.synchronize()
    saved = _os.environ.get("QGEMV_TILE")
    try:
        for spec in tiles:
            if spec == "default":
                _os.environ.pop("QGEMV_TILE", None)
            else:
                _os.environ["QGEMV_TILE"] = f"{fmt_name}:{spec}"
            for T in Ts:
                if call(T, 0) != _lib.QG_OK:
                    log(f"profile: {name} tile {spec} T={T} not run: {_lib.last_error()}")
                    continue
                for i in range(1, calls):
                    _lib.check(call(T, i), name)
                torch.cuda.synchronize()
                log(f"profile: {name} tile {spec} T={T}: {calls} calls")
    finally:
        if saved is None:
            _os.environ.pop("QGEMV_TILE", None)
        else:
            _os.environ["QGEMV_TILE"] = saved
    del ring


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget; 0 skips the CPU leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the timings of the other workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="N",
                    help="after the timed region, run N plain copies of the weight size (PMC calibration)")
    ap.add_argument("--profile", choices=PROFILE_WORKLOADS, metavar="WORKLOAD",
                    help="untimed calls of one workload for rocprofv3 (see --calls, --tiles); no JSON line")
    ap.add_argument("--calls", type=int, default=20, help="calls per T and tile with --profile")
    ap.add_argument("--tiles", default="default", help="space-separated QGEMV_TILE specs for --profile")
    ap.add_argument("--profile-t", default="1,2,3,4", help="comma-separated token counts for --profile")
    ap.add_argument("--bytes", type=int, default=0, help="algorithmic bytes per launch for --summarize-pmc")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM traffic table from two rocprofv3 --pmc runs of this script and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--skip-first", type=int, default=0,
                    help="with --summarize-trace: leave out the run's first N dispatches of this library")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="print per-kernel medians of every counter of a rocprofv3 --pmc run and exit")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.skip_first)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_pmc:
        fmt, rows, cols, _ = I.CONFIGS[WORKLOAD]
        summarize_pmc(*args.summarize_pmc, _lib.qg_packed_bytes(fmt, rows, cols), args.bytes or None)
        return

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} refused: only one GPU is measured "
              "(the mat-vec would shard by rows, one slab of W per GPU, with no collective)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    _lib.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.profile:
        Ts = tuple(int(t) for t in args.profile_t.split(","))
        if any(t < 1 or t > 4 for t in Ts):
            sys.exit("--profile-t: token counts are 1..4")
        profile_workload(torch, stream, args.profile, args.calls, args.tiles.split(), Ts)
        if args.copy_calibration:
            nb = _lib.qg_packed_bytes(I.FMT_Q8_0, 10240, 2560)
            src = torch.empty(nb // 4, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            for _ in range(args.copy_calibration):
                torch.mul(src, 1.0, out=dst)
            torch.cuda.synchronize()
        return

    case = I.dense_case(WORKLOAD)
    fmt, rows, cols = case["fmt"], case["rows"], case["cols"]
    nbytes = _lib.qg_packed_bytes(fmt, rows, cols)
    ring = ring_of(torch, case["W"])
    x_dev = torch.from_numpy(case["x"]).cuda()
    y_dev = torch.empty((4, rows), dtype=torch.float32, device="cuda")
    Ts = (1, 2, 3, 4)
    log(f"bench: {WORKLOAD} {nbytes} B/call, ring {len(ring)} copies, steps {args.steps}, warmup {args.warmup}")

    # settle: the same calls back to back for at least 0.2 s (and while one clock
    # sample is taken), so the timed region starts at the clocks sustained load
    # runs at (a fresh or idle GPU ramps its clocks up over the first
    # milliseconds); then the W warmup steps, then the timed steps
    def batch():
        for T in Ts:
            time_calls(torch, fmt, ring, x_dev[:T], rows, T, 25, stream, y_dev)
    clocks_before = clocks_under_load(torch, batch, 0.2)
    for T in Ts:
        time_calls(torch, fmt, ring, x_dev[:T], rows, T, args.warmup, stream, y_dev)
    torch.cuda.synchronize()

    # timed region: exactly K steps (K calls at each T), grouped by T
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs = {T: time_calls(torch, fmt, ring, x_dev[:T], rows, T, args.steps, stream, y_dev) for T in Ts}
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    clocks_after = clocks_under_load(torch, batch, 0.05)  # the same calls keep the GPU busy while sampled
    ms = {T: evs[T][0].elapsed_time(evs[T][1]) for T in Ts}
    total_ms = sum(ms.values())
    value = args.steps * len(Ts) * nbytes / (total_ms * 1e-3) / 1e9

    # after the timed region: 7 repeats per T (median, min, max of µs per call over
    # runs of >= 2 ms each) and a cache-warm figure (one buffer, 256 MB MALL-resident)
    reps = {}
    n_rep = max(20, int(2e3 / max(1e-3, min(ms.values()) * 1e3 / args.steps)))
    for T in Ts:
        vals = []
        for _ in range(7):
            s_, e_ = time_calls(torch, fmt, ring, x_dev[:T], rows, T, n_rep, stream, y_dev)
            torch.cuda.synchronize()
            vals.append(s_.elapsed_time(e_) * 1e3 / n_rep)
        s_, e_ = time_calls(torch, fmt, ring[:1], x_dev[:T], rows, T, n_rep, stream, y_dev)
        torch.cuda.synchronize()
        vals.sort()
        reps[T] = dict(median=round(vals[3], 3), min=round(vals[0], 3), max=round(vals[-1], 3),
                       warm_us=round(s_.elapsed_time(e_) * 1e3 / n_rep, 3), calls=n_rep)

    per_T = {}
    for T in Ts:
        us = ms[T] * 1e3 / args.steps
        per_T[str(T)] = dict(us_per_call=round(us, 3), gbs=round(nbytes / us / 1e3, 1),
                             pct_peak=round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1),
                             repeats_us=reps[T], tile=ops.query_tile("q8_0", rows, cols, T))
    dom = max(Ts, key=lambda T: ms[T])
    dom_us = ms[dom] * 1e3 / args.steps
    achieved = nbytes / dom_us / 1e3
    dom_kernel = kernel_name(ops.query_tile("q8_0", rows, cols, dom), dom)
    traffic = measured_traffic(dom_kernel)

    if args.copy_calibration:
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.copy_calibration):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    detail = {} if args.no_extra else other_workloads(torch, stream)
    if not args.no_extra:
        detail["hbm_read_probe"] = read_probe(torch, stream, nbytes)

    cpu = cpu_baseline(case, args.cpu_seconds) if args.cpu_seconds > 0 else None
    if cpu is not None and not args.no_extra:
        cpu["per_workload"] = cpu_baseline_per_workload()

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
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": dom_kernel, "T": dom, "us_per_launch": round(dom_us, 3),
                     "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "host": host_info(torch),
        "gpu_clocks": {"before_timed_region": clocks_before, "after_timed_region": clocks_after},
        "detail": detail,
        "wall_s_timed_region": round(wall_s, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
