#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X NVFP4 projection library.

One step = the weight-only NVFP4 projections of a 64-layer 27B-class decoder
at one row count: per layer qkv [12288x5120], o [5120x6144], the gate/up pair
2x[17408x5120] with SiLU*mul, down [5120x17408] (whose input is the pair's
output), 256 calls, 13,023,313,920 bytes of packed weights (E2M1 codes +
E4M3 scales, 9/16 byte per weight).  The calls run in order, each after the
previous one has completed, in shared launches of up to 40 calls.  Weights ~ N(0, 0.02^2) are drawn on the
device from seeded generators and quantized on the device; activations are
bf16 ~ N(0, 1).  All weights stay resident in HBM (no cache reuse between
layers: 13 GB >> the 256 MB Infinity Cache).

The headline value is the aggregate packed-weight read rate (GB/s) of the
rows=1 step; rows 2, 4, 8 are reported alongside.  Timing: W untimed warmup
steps, then K steps bracketed by device synchronization and HIP events on the
launch stream.  Each step is enqueued by one nvfp4_gemv_sequence call; the
roofline's kernel is its shared launch (bytes and duration per launch).  The
stand-alone gate/up pair launch (nvfp4_gemv_dual_silu) is timed as well, over
the 64 layers' pairs launched back to back.

The CPU baseline times the fp64 CPU oracle on layer 0 of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMV weight-read GB/s and % of HBM peak at rows=1 and rows=8"
HBM_PEAK_GBS = 8000.0
PAIR_NAME = "gate"
KERNEL_SOURCES = ("bit_weight_only_nvfp4_amd/csrc/nvfp4_stream.hip", "bit_weight_only_nvfp4_amd/csrc/nvfp4_core.h",
                  "bit_weight_only_nvfp4_amd/csrc/nvfp4_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_rows1_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def packed_weight_bytes(n: int, k: int) -> int:
    return n * k // 2 + n * k // 16


# packed weight bytes of one 64-layer decode step
STEP_BYTES_64 = 64 * (packed_weight_bytes(12288, 5120) + packed_weight_bytes(5120, 6144)
                      + 2 * packed_weight_bytes(17408, 5120) + packed_weight_bytes(5120, 17408))


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rows", default="1,2,4,8,16,32", help="row counts to time; the first is the headline")
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline duration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the lm-head, RMSNorm, MXFP4 and W8G32_F16S timings")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "LAUNCHES_PER_STEP"),
                    help="write the rows=1 decode-step kernel's HBM traffic per launch from two rocprofv3 "
                         "--pmc counter collections (FETCH_SIZE, WRITE_SIZE) of a --copy-calibration run of "
                         "the 64-layer sweep, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (known bytes) to scale PMC byte counters")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def build_sweep(nv, workloads, torch, dev, layers):
    qws = torch.empty(max(nv.nvfp4_quantize_workspace_bytes(n, k) for _, n, k in workloads.LAYER_PROJECTIONS),
                      dtype=torch.uint8, device=dev)
    mats = []
    for layer in range(layers):
        lm = {}
        for pi, (name, n, k) in enumerate(workloads.LAYER_PROJECTIONS):
            W = workloads.draw_weights_device(n, k, workloads.sweep_seed(layer, pi), dev)
            lm[name] = nv.nvfp4_quantize(W, workspace=qws)
            del W
        mats.append(lm)
    torch.cuda.synchronize()
    status = int(qws[:4].view(torch.int32).item())
    if status != 0:
        raise RuntimeError("device quantizer flagged a non-finite weight")
    return mats


def make_sequence(nv, torch, dev, workloads, mats, rows):
    x5120 = workloads.draw_x_device(rows, 5120, 5_000_000 + rows, dev)
    x6144 = workloads.draw_x_device(rows, 6144, 5_000_100 + rows, dev)
    y_qkv = torch.empty((rows, 12288), dtype=torch.bfloat16, device=dev)
    y_o = torch.empty((rows, 5120), dtype=torch.bfloat16, device=dev)
    o_gu = torch.empty((rows, 17408), dtype=torch.bfloat16, device=dev)
    y_down = torch.empty((rows, 5120), dtype=torch.bfloat16, device=dev)
    calls = []
    for lm in mats:
        calls.append((lm["qkv"], None, x5120, y_qkv))
        calls.append((lm["o"], None, x6144, y_o))
        calls.append((lm["gate"], lm["up"], x5120, o_gu))
        calls.append((lm["down"], None, o_gu, y_down))
    return nv.Sequence(calls)


def time_rows(torch, seq, ws, steps, warmup):
    """Average ms per step over `steps` steps after `warmup` untimed ones."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        seq.launch(ws)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        seq.launch(ws)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def time_pair(nv, torch, dev, mats, rows, ws, reps):
    """Average duration of one stand-alone gate/up pair launch (what
    nvfp4_gemv_dual_silu runs): the 64 layers' pairs back to back, one launch
    each (distinct weights, so no cache reuse), `reps` times, between HIP
    events on the launch stream."""
    x = torch.zeros((rows, 5120), dtype=torch.bfloat16, device=dev)
    o = torch.empty((rows, 17408), dtype=torch.bfloat16, device=dev)
    seq = nv.Sequence([(lm["gate"], lm["up"], x, o) for lm in mats])
    one_each = [None] * (2 * seq.n)   # event slots given: one launch per call
    seq.launch(ws, events=one_each)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        seq.launch(ws, events=one_each)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps / len(mats)


def cpu_baseline(workloads, torch, dev, target_s):
    import numpy as np

    import oracle

    oracle.build(force=False)
    q = {}
    nbytes = 0
    for pi, (name, n, k) in enumerate(workloads.LAYER_PROJECTIONS):
        W = workloads.draw_weights_device(n, k, workloads.sweep_seed(0, pi), dev).cpu().numpy()
        q[name] = oracle.quantize(W)
        nbytes += packed_weight_bytes(n, k)
        del W
    rng = np.random.default_rng(0)
    xs = {k: workloads.draw_x(rng, 1, k) for k in (5120, 6144, 17408)}
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemv(*q["qkv"], xs[5120])
        oracle.gemv(*q["o"], xs[6144])
        oracle.gemv_dual_silu(q["gate"], q["up"], xs[5120])
        oracle.gemv(*q["down"], xs[17408])
        passes += 1
        el = time.perf_counter() - t0
        if el >= target_s or el * (passes + 1) / passes > 30.0:
            break
    return {
        "value": round(nbytes * passes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "layer 0 of the decode-step sweep (qkv, o, gate/up pair with SiLU, down), rows=1, "
                  "fp64 CPU oracle (dequantize then dot), %d pass(es) in %.1f s, %d packed bytes per pass"
                  % (passes, el, nbytes),
    }


def load_traffic():
    """HBM bytes per launch of the rows=1 decode-step kernel (64-layer sweep)
    from the committed PMC summary, or None when it is missing or the kernel
    source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


STEP_KERNEL_TAG = "seq_kernel<1, true>"     # rows=1 shared-launch kernel of the decode step
COPY_BYTES = 1 << 30                         # --copy-calibration copies this many bytes


def summarize_pmc(fetch_csv, write_csv, launches_per_step):
    """HBM bytes per launch of the rows=1 decode-step kernel from rocprofv3
    counter collections.  FETCH_SIZE and WRITE_SIZE are reported in KiB per
    dispatch; each is scaled by what the same counter reads for the 1 GiB
    device copy of the same run (known bytes)."""
    import csv

    def per_kernel(path):
        out = {}
        for r in csv.DictReader(open(path)):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    f, w = per_kernel(fetch_csv), per_kernel(write_csv)

    def pick(table, pred):
        keys = [k for k in table if pred(k)]
        if not keys:
            raise SystemExit("no matching kernel in the counter file")
        vals = [v for k in keys for v in table[k]]
        return sum(vals) / len(vals), len(vals), keys[0]

    pair = lambda k: STEP_KERNEL_TAG in k
    # the 1 GiB device copy of --copy-calibration (the runtime's copy kernel)
    copy_f = max(v for k, vals in f.items() if "copyBuffer" in k for v in vals)
    copy_w = max(v for k, vals in w.items() if "copyBuffer" in k for v in vals)
    fetch_factor = COPY_BYTES / (copy_f * 1024.0)
    write_factor = COPY_BYTES / (copy_w * 1024.0)
    pf, n_f, name = pick(f, pair)
    pw, n_w, _ = pick(w, pair)
    fetch_bytes = pf * 1024.0 * fetch_factor
    write_bytes = pw * 1024.0 * write_factor
    t = {
        "kernel": name,
        "kernel_source_hash": kernel_source_hash(),
        "dispatches": [n_f, n_w],
        "fetch_kib_per_dispatch": round(pf, 1),
        "write_kib_per_dispatch": round(pw, 1),
        "copy_fetch_kib": round(copy_f, 1),
        "copy_write_kib": round(copy_w, 1),
        "fetch_factor": round(fetch_factor, 4),
        "write_factor": round(write_factor, 4),
        "launches_per_step": launches_per_step,
        "algorithmic_bytes_per_launch": STEP_BYTES_64 // launches_per_step,
        "bytes_per_launch": int(round(fetch_bytes + write_bytes)),
    }
    with open(TRAFFIC_FILE, "w") as fo:
        json.dump(t, fo, indent=1)
    print(json.dumps(t))


DENSE_N, DENSE_K = 151936, 5120   # an lm head of a vocabulary-sized n (the pages give no vocabulary size)


def time_dense(nv, torch, dev, rows_list, reps):
    """The dense bf16 projection (nvfp4_dense_gemv_bf16) on a [151936 x 5120]
    bf16 lm head: average duration of `reps` back-to-back calls (1.56 GB of
    weights: nothing stays cached between them) between HIP events, per row
    count; GB/s counts the weight bytes once per call."""
    g = torch.Generator(device=dev).manual_seed(4321)
    W = (torch.randn((DENSE_N, DENSE_K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    wbytes = DENSE_N * DENSE_K * 2
    out = {"shape": [DENSE_N, DENSE_K], "weight_bytes": wbytes, "by_rows": {}}
    stream = torch.cuda.current_stream()
    for r in rows_list:
        x = torch.randn((r, DENSE_K), generator=g, device=dev).to(torch.bfloat16)
        y = torch.empty((r, DENSE_N), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            nv.nvfp4_dense_gemv_bf16(W, x, out=y)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            nv.nvfp4_dense_gemv_bf16(W, x, out=y)
        stop.record(stream)
        torch.cuda.synchronize()
        us = start.elapsed_time(stop) * 1e3 / reps
        gbs = wbytes / (us * 1e-6) / 1e9
        out["by_rows"][str(r)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                  "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        log("dense lm head %dx%d bf16, rows=%d: %.2f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (
            DENSE_N, DENSE_K, r, us, gbs, 100 * gbs / HBM_PEAK_GBS))
    del W
    return out


def time_mx(nv, torch, dev, rows_list, reps):
    """The MXFP4 projection (nvfp4_mxfp4_gemv) on an lm-head-sized [151936 x
    5120] and a gate-sized [17408 x 5120] matrix: random codes and E8M0 scale
    bytes 118..124 drawn on the device (any bytes are valid MXFP4), back-to-back
    calls between HIP events; GB/s counts codes + scales once per call."""
    g = torch.Generator(device=dev).manual_seed(2024)
    out = {}
    stream = torch.cuda.current_stream()
    for n, k in ((151936, 5120), (17408, 5120)):
        codes = torch.randint(0, 256, (n, k // 2), generator=g, device=dev, dtype=torch.uint8)
        scales = torch.randint(118, 125, (n, k // 32), generator=g, device=dev, dtype=torch.uint8)
        wbytes = n * k // 2 + n * k // 32
        res = {"shape": [n, k], "weight_bytes": wbytes, "by_rows": {}}
        for r in rows_list:
            x = torch.randn((r, k), generator=g, device=dev).to(torch.bfloat16)
            y = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                nv.nvfp4_mxfp4_gemv(codes, scales, x, out=y)
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(reps):
                nv.nvfp4_mxfp4_gemv(codes, scales, x, out=y)
            stop.record(stream)
            torch.cuda.synchronize()
            us = start.elapsed_time(stop) * 1e3 / reps
            gbs = wbytes / (us * 1e-6) / 1e9
            res["by_rows"][str(r)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                      "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
            log("mxfp4 %dx%d rows=%d: %.2f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (
                n, k, r, us, gbs, 100 * gbs / HBM_PEAK_GBS))
        out["%dx%d" % (n, k)] = res
        del codes, scales
    return out


def time_w8(nv, torch, dev, rows_list, reps):
    """The W8G32_F16S projection (nvfp4_w8g32_gemv) on a gate-sized [17408 x
    5120] and a down-sized [5120 x 17408] matrix: random int8 codes and fp16
    scales 2^-8..2^-6 drawn on the device, back-to-back calls between HIP
    events; GB/s counts codes + scales once per call."""
    g = torch.Generator(device=dev).manual_seed(2025)
    out = {}
    stream = torch.cuda.current_stream()
    for n, k in ((17408, 5120), (5120, 17408)):
        codes = torch.randint(-127, 128, (n, k), generator=g, device=dev, dtype=torch.int8)
        scales = torch.exp2(torch.randint(-8, -5, (n, k // 32), generator=g, device=dev).float()).half()
        wbytes = n * k + n * k // 32 * 2
        res = {"shape": [n, k], "weight_bytes": wbytes, "by_rows": {}}
        for r in rows_list:
            x = torch.randn((r, k), generator=g, device=dev).to(torch.bfloat16)
            y = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                nv.nvfp4_w8g32_gemv(codes, scales, x, out=y)
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(reps):
                nv.nvfp4_w8g32_gemv(codes, scales, x, out=y)
            stop.record(stream)
            torch.cuda.synchronize()
            us = start.elapsed_time(stop) * 1e3 / reps
            gbs = wbytes / (us * 1e-6) / 1e9
            res["by_rows"][str(r)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                      "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
            log("w8g32 %dx%d rows=%d: %.2f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (
                n, k, r, us, gbs, 100 * gbs / HBM_PEAK_GBS))
        out["%dx%d" % (n, k)] = res
        del codes, scales
    return out


def time_norm(nv, torch, dev, reps):
    """nvfp4_residual_rmsnorm at the 27B model's hidden size (k = 5120): the
    average call at decode row counts (1 and 8: a few tens of KB, bound by
    latency) and GB/s at 4096 rows (reads residual and delta, writes
    residual_out and x: 8 bytes per element)."""
    g = torch.Generator(device=dev).manual_seed(99)
    k = 5120
    w = torch.randn((k,), generator=g, device=dev).to(torch.bfloat16)
    out = {"k": k, "by_rows": {}}
    stream = torch.cuda.current_stream()
    for rows in (1, 8, 4096):
        r = torch.randn((rows, k), generator=g, device=dev).to(torch.bfloat16)
        h = torch.randn((rows, k), generator=g, device=dev).to(torch.bfloat16)
        ro, x = torch.empty_like(r), torch.empty_like(r)
        for _ in range(3):
            nv.nvfp4_residual_rmsnorm(r, h, w, residual_out=ro, x=x)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            nv.nvfp4_residual_rmsnorm(r, h, w, residual_out=ro, x=x)
        stop.record(stream)
        torch.cuda.synchronize()
        us = start.elapsed_time(stop) * 1e3 / reps
        gbs = rows * k * 8 / (us * 1e-6) / 1e9
        out["by_rows"][str(rows)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                     "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        log("residual add + RMSNorm k=%d rows=%d: %.2f us, %.1f GB/s" % (k, rows, us, gbs))
    return out


def main():
    args = parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], int(args.summarize_pmc[2]))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the NVFP4 projection path here has no multi-GPU mode "
              "(asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_weight_only_nvfp4_amd as nv
    import workloads

    nv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows_list = [int(r) for r in args.rows.split(",")]

    t0 = time.time()
    mats = build_sweep(nv, workloads, torch, dev, args.layers)
    layer_bytes = sum(packed_weight_bytes(n, k) for _, n, k in workloads.LAYER_PROJECTIONS)
    step_bytes = layer_bytes * args.layers
    pair_bytes = 2 * packed_weight_bytes(17408, 5120)
    log("sweep built: %d layers, %d packed weight bytes per step (%.1f s)" % (args.layers, step_bytes,
                                                                             time.time() - t0))

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 1 GiB device-to-device copy done")

    seqs = {r: make_sequence(nv, torch, dev, workloads, mats, r) for r in rows_list}
    ws = torch.zeros(max(s.workspace_bytes for s in seqs.values()), dtype=torch.uint8, device=dev)
    by_rows = {}
    for r in rows_list:
        ms = time_rows(torch, seqs[r], ws, args.steps, args.warmup)
        pair_ms = time_pair(nv, torch, dev, mats, r, ws, max(2, args.steps // 10))
        gbs = step_bytes / (ms * 1e-3) / 1e9
        by_rows[str(r)] = {
            "ms_per_step": round(ms, 4),
            "launches_per_step": seqs[r].launches,
            "GB_per_s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "gate_up_pair_us": round(pair_ms * 1e3, 3),
            "gate_up_pair_GB_per_s": round(pair_bytes / (pair_ms * 1e-3) / 1e9, 1),
        }
        log("rows=%d: %.4f ms/step in %d launches, %.1f GB/s (%.1f%% of 8 TB/s); stand-alone gate/up pair "
            "%.2f us" % (r, ms, seqs[r].launches, gbs, 100 * gbs / HBM_PEAK_GBS, pair_ms * 1e3))

    head = by_rows[str(rows_list[0])]
    # The dominant kernel is the shared launch that runs the step's calls
    # (every byte of the step is read by it): bytes and duration per launch.
    launches = head["launches_per_step"]
    launch_bytes = step_bytes / launches
    launch_us = head["ms_per_step"] * 1e3 / launches
    achieved = launch_bytes / (launch_us * 1e-6) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": "seq_kernel<%d, true> (shared launch of %d consecutive decode-step calls: qkv, o, "
                  "gate/up pair + SiLU*mul, down)" % (rows_list[0], round(4 * args.layers / launches)),
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": load_traffic() if args.layers == 64 and rows_list[0] == 1 else None,
        "bytes_per_launch": round(launch_bytes),
        "avg_launch_us": round(launch_us, 2),
    }

    dense = None
    if not args.no_dense:
        dense = time_dense(nv, torch, dev, [r for r in (1, 8) if r in rows_list] or [rows_list[0]],
                           max(5, args.steps // 5))

    norm = None if args.no_dense else time_norm(nv, torch, dev, max(10, args.steps // 2))
    # calls of 25-150 us: enough back-to-back calls that launch start-up is a small share
    mx = None if args.no_dense else time_mx(nv, torch, dev, [r for r in (1, 8) if r in rows_list] or [rows_list[0]],
                                            max(50, args.steps))
    w8 = None if args.no_dense else time_w8(nv, torch, dev, [r for r in (1, 8) if r in rows_list] or [rows_list[0]],
                                            max(50, args.steps))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on layer 0 ...")
        cpu = cpu_baseline(workloads, torch, dev, args.cpu_seconds)
        log("cpu baseline: %.3f GB/s on %d threads" % (cpu["value"], cpu["cores"]))

    line = {
        "metric": METRIC,
        "value": head["GB_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0,0.02^2) weights quantized to NVFP4 on the device, bf16 N(0,1) activations",
        "config": {
            "workload": "64-layer decode-step sweep: per layer qkv 12288x5120, o 5120x6144, gate/up pair "
                        "2x17408x5120 + SiLU*mul, down 5120x17408; rows=%d" % rows_list[0],
            "layers": args.layers,
            "rows": rows_list[0],
            "packed_weight_bytes_per_step": step_bytes,
            "calls_per_step": 4 * args.layers,
            "launches_per_step": head["launches_per_step"],
        },
        "pct_hbm_peak": head["pct_hbm_peak"],
        "by_rows": by_rows,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_lm_head": dense,
        "residual_rmsnorm": norm,
        "mxfp4": mx,
        "w8g32_f16s": w8,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
