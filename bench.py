#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X NVFP4 projection library.

One step = the weight-only NVFP4 projections of a 64-layer 27B-class decoder
at one row count: per layer qkv [12288x5120], o [5120x6144], the gate/up pair
2x[17408x5120] with SiLU*mul, down [5120x17408] (whose input is the pair's
output), 256 calls, 13,023,313,920 bytes of packed weights (E2M1 codes +
E4M3 scales, 9/16 byte per weight), in one shared launch.  The calls compute
what they would one by one; a call waits for the calls before it where it
depends on one: down reads the pair's output (one wait per layer; the pair's
output alternates between two buffers, so the next layer's pair does not wait
for this layer's down to finish reading it).  Weights ~ N(0, 0.02^2) are drawn on the
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

After timing, every row count's workspace wait flag must be clear, and at
rows 1 and 8 sampled outputs of the timed step's last layer (every call of
layer 63, 256 features each) are checked against the CPU oracle.

The same step with each layer's two residual add + RMSNorm calls (the first
producing qkv's input from the residual and the previous layer's down output,
the second the pair's input from the residual and o's output) fused into its
launches is timed at rows 1 and 8 as well (step_with_norms).

Single projection calls (qkv at 1 row, the gate/up pair at 1 row, down at 8
rows with 1% outlier groups) are timed one call between two events each,
rotating over at least 1 GiB of distinct packed weights, and reported as
median / p10 / p90 beside the streaming-read ceiling for the same bytes.

The CPU baseline times the CPU oracle on layer 0 of the same workload at all
host threads and at one thread.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import platform
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_traffic.json")


def _code_tokens(text: str) -> str:
    """C++ source without its comments and with whitespace collapsed, so that
    editing a comment does not make the traffic counters stale.  String and
    character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the decode-step kernel's code (comments and layout ignored)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_tokens(f.read()).encode())
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
    ap.add_argument("--step-only", action="store_true",
                    help="time the decode step alone, for profiling: no stand-alone pair, norm-step, read-ceiling, "
                         "single-call or format timings (their launches would mix with the step's in a profile)")
    ap.add_argument("--long-call-only", action="store_true",
                    help="time the long [65536 x 16384] call alone at the --rows row counts, for profiling the "
                         "tile loop without the decode step's per-call work; prints its figures as JSON")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("RDREQ_CSV", "WRITE_CSV", "LAUNCHES_PER_STEP"),
                    help="write the decode-step kernels' HBM traffic per launch from two rocprofv3 --pmc counter "
                         "collections (TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_128B_sum TCC_EA0_RDREQ_64B_sum "
                         "TCC_EA0_RDREQ_32B_sum; WRITE_SIZE) of a --copy-calibration run of the 64-layer sweep, "
                         "then exit")
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


def make_sequence(nv, torch, dev, workloads, mats, rows, bufs=None, norms=False):
    """The decode step's calls for every layer: qkv, o, the gate/up pair and
    down (fed by the pair).  The pair's output alternates between two buffers
    from layer to layer, so that a pair never overwrites what the previous
    layer's down still reads: down waits for its own layer's pair only (one
    wait per layer).  With norms, each layer also runs its two residual add +
    RMSNorm calls inside the same launches: the first (residual += previous
    down output) produces qkv's input, the second (residual += o's output) the
    pair's."""
    x5120 = workloads.draw_x_device(rows, 5120, 5_000_000 + rows, dev)
    x6144 = workloads.draw_x_device(rows, 6144, 5_000_100 + rows, dev)
    y_qkv = torch.empty((rows, 12288), dtype=torch.bfloat16, device=dev)
    y_o = torch.zeros((rows, 5120), dtype=torch.bfloat16, device=dev)
    o_gus = [torch.empty((rows, 17408), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    y_down = torch.zeros((rows, 5120), dtype=torch.bfloat16, device=dev)
    calls = []
    if norms:
        resid = workloads.draw_x_device(rows, 5120, 5_000_200 + rows, dev)
        g = torch.Generator(device=dev).manual_seed(5_000_300)
        lns = (torch.randn((len(mats), 2, 5120), generator=g, device=dev) * 0.1).to(torch.bfloat16)
    for li, lm in enumerate(mats):
        if norms:
            calls.append(nv.Norm(resid, y_down, lns[li, 0], x5120, gemma_offset=True))
        calls.append((lm["qkv"], None, x5120, y_qkv))
        calls.append((lm["o"], None, x6144, y_o))
        if norms:
            calls.append(nv.Norm(resid, y_o, lns[li, 1], x5120, gemma_offset=True))
        o_gu = o_gus[li % 2]
        calls.append((lm["gate"], lm["up"], x5120, o_gu))
        calls.append((lm["down"], None, o_gu, y_down))
    if bufs is not None:
        # the last layer's buffers (the parity sample checks that layer)
        bufs.update(x5120=x5120, x6144=x6144, y_qkv=y_qkv, y_o=y_o, o_gu=o_gus[(len(mats) - 1) % 2], y_down=y_down)
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(workloads, torch, dev, target_s):
    """The CPU oracle (fp64 dequantize-then-dot, OpenMP over output features)
    on layer 0 of the sweep at rows=1: all host threads over the whole layer,
    and one thread over its qkv projection; GB/s of the same packed bytes."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    q = {}
    for pi, (name, n, k) in enumerate(workloads.LAYER_PROJECTIONS):
        W = workloads.draw_weights_device(n, k, workloads.sweep_seed(0, pi), dev).cpu().numpy()
        q[name] = oracle.quantize(W)
        del W
    rng = np.random.default_rng(0)
    xs = {k: workloads.draw_x(rng, 1, k) for k in (5120, 6144, 17408)}
    layer_bytes = sum(packed_weight_bytes(n, k) for _, n, k in workloads.LAYER_PROJECTIONS)
    qkv_bytes = packed_weight_bytes(12288, 5120)

    def run(threads, fn, nbytes, budget):
        oracle.set_num_threads(threads)
        passes, t0 = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget or el * (passes + 1) / passes > 2.5 * budget:
                break
        return nbytes * passes / el / 1e9, passes, el

    def layer():
        oracle.gemv(*q["qkv"], xs[5120])
        oracle.gemv(*q["o"], xs[6144])
        oracle.gemv_dual_silu(q["gate"], q["up"], xs[5120])
        oracle.gemv(*q["down"], xs[17408])

    all_threads = os.cpu_count() or 1
    gbs_all, p_all, el_all = run(all_threads, layer, layer_bytes, target_s)
    gbs_one, p_one, el_one = run(1, lambda: oracle.gemv(*q["qkv"], xs[5120]), qkv_bytes, target_s / 2)
    oracle.set_num_threads(all_threads)
    return {
        "value": round(gbs_all, 4),
        "unit": "GB/s",
        "cores": all_threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": "layer 0 of the decode-step sweep (qkv, o, gate/up pair with SiLU, down), rows=1, fp64 CPU "
                  "oracle (dequantize then dot), %d thread(s), %d pass(es) in %.1f s, %d packed bytes per pass"
                  % (all_threads, p_all, el_all, layer_bytes),
        "one_thread": {"value": round(gbs_one, 5), "unit": "GB/s", "cores": 1,
                       "sample": "qkv projection of layer 0 [12288 x 5120], rows=1, %d pass(es) in %.1f s"
                                 % (p_one, el_one)},
    }


def parity_sample(nv, torch, mats, bufs, rows, nsel=256, seed=7):
    """Sampled outputs of the last layer of the timed step (every call of
    layer 63: qkv, o, the gate/up pair, down -- whose activations are the
    pair's outputs of the same step) against the CPU oracle: the bf16 outputs
    within 1e-3 * sum|w*x| plus half a bf16 ulp of the oracle's fp64 value, and
    within one bf16 ulp of its bf16 value wherever |y| >= 2^-12 sum|w*x|."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    lm = mats[-1]
    rng = np.random.default_rng(seed)

    def host_weight(w):
        c, s_, g = nv.nvfp4_unpack(w)
        return c.cpu().numpy(), s_.cpu().numpy(), np.float32(g.item())

    def bits(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)

    def val(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    worst = {"max_err_over_absdot": 0.0, "max_bf16_ulp": 0, "outputs": 0, "exempt": 0}

    def compare(out16, ref, absd, ref16):
        y = val(out16)
        err = np.abs(y - ref)
        bound = 1e-3 * absd + np.abs(ref) * 2.0 ** -8
        if not np.all(err <= bound):
            raise SystemExit("parity sample failed at rows=%d: max err/bound %.3g" % (rows, (err / bound).max()))
        enforce = np.abs(ref) >= 2.0 ** -12 * absd
        dist = np.abs(ordered(out16) - ordered(ref16))
        if np.any(dist[enforce] > 1):
            raise SystemExit("parity sample failed at rows=%d: %d bf16 outputs > 1 ulp" % (rows, int(np.sum(dist[enforce] > 1))))
        worst["max_err_over_absdot"] = max(worst["max_err_over_absdot"],
                                           float(np.max(err / np.where(absd > 0, absd, 1.0))))
        worst["max_bf16_ulp"] = max(worst["max_bf16_ulp"], int(dist[enforce].max()) if enforce.any() else 0)
        worst["outputs"] += int(out16.size)
        worst["exempt"] += int(np.sum(~enforce))

    x5120, x6144 = bits(bufs["x5120"]), bits(bufs["x6144"])
    for name, x, yb in (("qkv", x5120, bufs["y_qkv"]), ("o", x6144, bufs["y_o"])):
        w = host_weight(lm[name])
        sel = np.sort(rng.choice(lm[name].n, nsel, replace=False))
        ref, absd, ref16 = oracle.gemv(*w, x, sel=sel)
        compare(bits(yb)[:, sel], ref, absd, ref16)
    g, u = host_weight(lm["gate"]), host_weight(lm["up"])
    sel = np.sort(rng.choice(lm["gate"].n, nsel, replace=False))
    d = oracle.gemv_dual_silu(g, u, x5120, sel=sel)
    o16 = bits(bufs["o_gu"])
    y = val(o16[:, sel])
    err = np.abs(y - d["o"])
    from oracle import check
    bound = check.dual_bound(d) + np.abs(d["o"]) * 2.0 ** -8
    if not np.all(err <= bound):
        raise SystemExit("parity sample failed at rows=%d (gate/up pair)" % rows)
    worst["outputs"] += int(y.size)
    w = host_weight(lm["down"])
    sel = np.sort(rng.choice(lm["down"].n, nsel, replace=False))
    ref, absd, ref16 = oracle.gemv(*w, o16, sel=sel)
    compare(bits(bufs["y_down"])[:, sel], ref, absd, ref16)
    worst["max_err_over_absdot"] = float("%.3g" % worst["max_err_over_absdot"])
    worst["features_per_call"] = nsel
    worst["layer"] = len(mats) - 1
    return worst


def pctl(vals, p):
    import numpy as np
    return float(np.percentile(np.asarray(vals, dtype=np.float64), p))


def time_calls(torch, launch, ncalls, warmup=20):
    """Per-call device time: every call between two events of its own, all
    enqueued before one synchronization.  Returns the durations in us."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ncalls)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        launch(i)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def call_stats(us, nbytes, copies):
    med = pctl(us, 50)
    return {"calls": len(us), "copies": copies, "bytes_per_call": nbytes,
            "bytes_rotated": nbytes * copies,
            "median_us": round(med, 3), "p10_us": round(pctl(us, 10), 3), "p90_us": round(pctl(us, 90), 3),
            "GB_per_s_median": round(nbytes / (med * 1e-6) / 1e9, 1),
            "pct_hbm_peak_median": round(100 * nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}


CEILING_BYTES = 1 << 31     # the read-ceiling buffer: 2 GiB, far beyond the 256 MB Infinity Cache


def read_ceiling(nv, torch, dev, buf, nbytes, ncalls):
    """Per-call durations of the streaming-read kernel over nbytes (at most
    half the 2 GiB buffer), rotating the start offset through the buffer."""
    if not 0 < nbytes <= CEILING_BYTES // 2:
        raise ValueError("read ceiling of %d bytes: at most %d" % (nbytes, CEILING_BYTES // 2))
    span = (CEILING_BYTES - nbytes) // 4096 * 4096
    offs = [(i * 1_000_003 * 4096) % max(span, 4096) if span > 0 else 0 for i in range(ncalls + 20)]
    sink = torch.empty(256, dtype=torch.int32, device=dev)
    return time_calls(torch, lambda i: nv.nvfp4_read_ceiling(buf, nbytes, sink, offset=offs[i % len(offs)]),
                      ncalls)


def single_calls(nv, torch, dev, workloads, mats, ceil_buf, ncalls=200):
    """The single-call configurations, one call between two events each,
    rotating over >= 1 GiB of distinct packed weights: qkv [12288 x 5120] at
    1 row (the sweep's 64 qkv weights), the gate/up pair 2 x [17408 x 5120] at
    1 row (the sweep's 64 pairs), down [5120 x 17408] at 8 rows with 1% of its
    16-weight groups x50 (22 weights drawn and quantized for this).  Beside
    each, the read ceiling for the same bytes."""
    out = {}
    x1 = workloads.draw_x_device(1, 5120, 6_000_001, dev)
    y_qkv = torch.empty((1, 12288), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(nv.nvfp4_workspace_bytes(12288, 5120, 1), 16), dtype=torch.uint8, device=dev)
    qkv = [lm["qkv"] for lm in mats]
    nb = packed_weight_bytes(12288, 5120)
    us = time_calls(torch, lambda i: nv.nvfp4_gemv(qkv[i % len(qkv)], x1, out=y_qkv, workspace=ws), ncalls)
    out["qkv_12288x5120_rows1"] = call_stats(us, nb, len(qkv))
    out["qkv_12288x5120_rows1"]["read_ceiling_median_us"] = round(pctl(read_ceiling(nv, torch, dev, ceil_buf, nb, ncalls), 50), 3)

    o_gu = torch.empty((1, 17408), dtype=torch.bfloat16, device=dev)
    ws2 = torch.zeros(max(nv.nvfp4_workspace_bytes(17408, 5120, 1, True), 16), dtype=torch.uint8, device=dev)
    nb2 = 2 * packed_weight_bytes(17408, 5120)
    us = time_calls(torch, lambda i: nv.nvfp4_gemv_dual_silu(mats[i % len(mats)]["gate"], mats[i % len(mats)]["up"],
                                                              x1, out=o_gu, workspace=ws2), ncalls)
    out["gate_up_2x17408x5120_rows1"] = call_stats(us, nb2, len(mats))
    out["gate_up_2x17408x5120_rows1"]["read_ceiling_median_us"] = round(pctl(read_ceiling(nv, torch, dev, ceil_buf, nb2, ncalls), 50), 3)

    n, k = 5120, 17408
    ncopies = -(-(1 << 30) // packed_weight_bytes(n, k))
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    downs = []
    for c in range(ncopies):
        g = torch.Generator(device=dev).manual_seed(7_000_000 + c)
        W = torch.randn((n, k), generator=g, device=dev, dtype=torch.float32).mul_(workloads.WEIGHT_STD)
        ngroups = n * k // workloads.GROUP
        idx = torch.randperm(ngroups, generator=g, device=dev)[: round(0.01 * ngroups)]
        W.view(ngroups, workloads.GROUP)[idx] *= 50.0
        downs.append(nv.nvfp4_quantize(W, workspace=qws))
        del W, idx
    x8 = workloads.draw_x_device(8, k, 6_000_008, dev)
    y8 = torch.empty((8, n), dtype=torch.bfloat16, device=dev)
    ws3 = torch.zeros(max(nv.nvfp4_workspace_bytes(n, k, 8), 16), dtype=torch.uint8, device=dev)
    nb3 = packed_weight_bytes(n, k)
    us = time_calls(torch, lambda i: nv.nvfp4_gemv(downs[i % ncopies], x8, out=y8, workspace=ws3), ncalls)
    out["down_5120x17408_rows8_outliers"] = call_stats(us, nb3, ncopies)
    out["down_5120x17408_rows8_outliers"]["read_ceiling_median_us"] = round(pctl(read_ceiling(nv, torch, dev, ceil_buf, nb3, ncalls), 50), 3)
    for key, floor in (("qkv_12288x5120_rows1", 5.90), ("gate_up_2x17408x5120_rows1", 16.71),
                       ("down_5120x17408_rows8_outliers", 8.95)):
        out[key]["derived_floor_us"] = floor
        out[key]["pct_of_read_ceiling"] = round(100 * out[key]["read_ceiling_median_us"] / out[key]["median_us"], 1)
    del downs
    return out


def load_traffic(rows):
    """HBM bytes per launch of the decode-step kernel at `rows` (64-layer
    sweep) from the committed PMC summary, or None when it is missing or the
    kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("by_rows", {}).get(str(rows), {}).get("bytes_per_launch")


COPY_BYTES = 1 << 30                         # --copy-calibration copies this many bytes


def summarize_pmc(rdreq_csv, write_csv, launches_per_step):
    """HBM bytes per launch of the decode-step kernels (seq_kernel<R, true>)
    from two rocprofv3 counter collections of a --copy-calibration run: read
    bytes from the L2-to-memory read requests by size (TCC_EA0_RDREQ_128B /
    _64B / _32B, x 128 / 64 / 32 bytes), write bytes from WRITE_SIZE (KiB).
    Both are checked against the 1 GiB device copy of the same run (known
    bytes), and scaled by it.  FETCH_SIZE is not used: its expression counts
    a 128-byte read request as 64 bytes on this GPU (it reads half the copy's
    bytes), while the 128-byte request count gives the copy's size exactly."""
    import csv

    def dispatches(path):
        out = {}
        for r in csv.DictReader(open(path)):
            d = out.setdefault(r["Dispatch_Id"], {"kernel": r["Kernel_Name"]})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
        return list(out.values())

    rd, wr = dispatches(rdreq_csv), dispatches(write_csv)

    def read_bytes(d):
        return (128 * d["TCC_EA0_RDREQ_128B_sum"] + 64 * d["TCC_EA0_RDREQ_64B_sum"]
                + 32 * d["TCC_EA0_RDREQ_32B_sum"])

    copy_r = max(read_bytes(d) for d in rd if "copyBuffer" in d["kernel"])
    copy_w = max(d["WRITE_SIZE"] for d in wr if "copyBuffer" in d["kernel"]) * 1024.0
    read_factor, write_factor = COPY_BYTES / copy_r, COPY_BYTES / copy_w
    t = {"kernel_source_hash": kernel_source_hash(), "copy_read_bytes": int(copy_r), "copy_write_bytes": int(copy_w),
         "read_factor": round(read_factor, 4), "write_factor": round(write_factor, 4),
         "launches_per_step": launches_per_step, "algorithmic_bytes_per_launch": STEP_BYTES_64 // launches_per_step,
         "by_rows": {}}
    for rows in (1, 2, 4, 8, 16):
        tag = "seq_kernel<%d, true>" % rows
        r = [read_bytes(d) for d in rd if tag in d["kernel"]]
        w = [d["WRITE_SIZE"] * 1024.0 for d in wr if tag in d["kernel"]]
        if not r or not w:
            continue
        rb, wb = sum(r) / len(r) * read_factor, sum(w) / len(w) * write_factor
        t["by_rows"][str(rows)] = {"dispatches": [len(r), len(w)], "read_bytes_per_launch": int(round(rb)),
                                   "write_bytes_per_launch": int(round(wb)), "bytes_per_launch": int(round(rb + wb)),
                                   "ratio_to_algorithmic": round((rb + wb) / (STEP_BYTES_64 / launches_per_step), 4)}
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


ROTATE_BYTES = 1 << 30   # distinct bytes cycled through by back-to-back timings (>= 4x the 256 MB Infinity Cache)


def time_rotating(torch, launch, copies, reps):
    """Average us per call of `reps` back-to-back calls cycling through
    `copies` distinct operand sets (launch(i) runs set i % copies)."""
    stream = torch.cuda.current_stream()
    for i in range(min(copies, 3)):
        launch(i)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(reps):
        launch(i % copies)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e3 / reps


def time_long_call(nv, torch, dev, workloads, rows_list, reps, ceil_buf):
    """One long projection call, [65536 x 16384] (604 MB packed, 512 strips of
    64 super-tiles: two whole strips per workgroup, no split-K), back to back
    over two distinct copies (1.2 GB): the tile loop's own streaming rate,
    without the per-call and per-wait costs of the decode step's short calls;
    beside it the read ceiling for the same bytes."""
    n, k = 65536, 16384
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    mats = []
    for c in range(2):
        W = workloads.draw_weights_device(n, k, 6_000_000 + c, dev)
        mats.append(nv.nvfp4_quantize(W, workspace=qws))
        del W
    del qws
    nb = packed_weight_bytes(n, k)
    ceil_us = pctl(read_ceiling(nv, torch, dev, ceil_buf, nb, 20), 50)
    res = {"shape": [n, k], "packed_bytes": nb, "copies": len(mats), "read_ceiling_us": round(ceil_us, 2),
           "by_rows": {}}
    for r in rows_list:
        x = workloads.draw_x_device(r, k, 6_000_100 + r, dev)
        y = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
        us = time_rotating(torch, lambda i: nv.nvfp4_gemv(mats[i], x, out=y), len(mats), reps)
        gbs = nb / (us * 1e-6) / 1e9
        res["by_rows"][str(r)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                  "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                                  "pct_of_read_ceiling": round(100 * ceil_us / us, 1)}
        log("long call %dx%d rows=%d: %.2f us, %.1f GB/s (%.1f%% of 8 TB/s, %.1f%% of the read ceiling)"
            % (n, k, r, us, gbs, 100 * gbs / HBM_PEAK_GBS, 100 * ceil_us / us))
    del mats
    return res


def time_mx(nv, torch, dev, rows_list, reps):
    """The MXFP4 projection (nvfp4_mxfp4_gemv) on an lm-head-sized [151936 x
    5120] and a gate-sized [17408 x 5120] matrix: random codes and E8M0 scale
    bytes 118..124 drawn on the device (any bytes are valid MXFP4), back-to-back
    calls cycling through >= 1 GiB of distinct copies; GB/s counts codes +
    scales once per call."""
    g = torch.Generator(device=dev).manual_seed(2024)
    out = {}
    for n, k in ((151936, 5120), (17408, 5120)):
        wbytes = n * k // 2 + n * k // 32
        copies = -(-ROTATE_BYTES // wbytes)
        cs = [(torch.randint(0, 256, (n, k // 2), generator=g, device=dev, dtype=torch.uint8),
               torch.randint(118, 125, (n, k // 32), generator=g, device=dev, dtype=torch.uint8))
              for _ in range(copies)]
        res = {"shape": [n, k], "weight_bytes": wbytes, "copies": copies, "by_rows": {}}
        for r in rows_list:
            x = torch.randn((r, k), generator=g, device=dev).to(torch.bfloat16)
            y = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
            us = time_rotating(torch, lambda i: nv.nvfp4_mxfp4_gemv(cs[i][0], cs[i][1], x, out=y), copies,
                               max(reps, 3 * copies))
            gbs = wbytes / (us * 1e-6) / 1e9
            res["by_rows"][str(r)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                      "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
            log("mxfp4 %dx%d rows=%d (%d copies): %.2f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (
                n, k, r, copies, us, gbs, 100 * gbs / HBM_PEAK_GBS))
        out["%dx%d" % (n, k)] = res
        del cs
    return out


def time_w8(nv, torch, dev, rows_list, reps):
    """The W8G32_F16S projection (nvfp4_w8g32_gemv) on a gate-sized [17408 x
    5120] and a down-sized [5120 x 17408] matrix: random int8 codes and fp16
    scales 2^-8..2^-6 drawn on the device, back-to-back calls cycling through
    >= 1 GiB of distinct copies; GB/s counts codes + scales once per call."""
    g = torch.Generator(device=dev).manual_seed(2025)
    out = {}
    for n, k in ((17408, 5120), (5120, 17408)):
        wbytes = n * k + n * k // 32 * 2
        copies = -(-ROTATE_BYTES // wbytes)
        cs = [(torch.randint(-127, 128, (n, k), generator=g, device=dev, dtype=torch.int8),
               torch.exp2(torch.randint(-8, -5, (n, k // 32), generator=g, device=dev).float()).half())
              for _ in range(copies)]
        res = {"shape": [n, k], "weight_bytes": wbytes, "copies": copies, "by_rows": {}}
        for r in rows_list:
            x = torch.randn((r, k), generator=g, device=dev).to(torch.bfloat16)
            y = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
            us = time_rotating(torch, lambda i: nv.nvfp4_w8g32_gemv(cs[i][0], cs[i][1], x, out=y), copies,
                               max(reps, 3 * copies))
            gbs = wbytes / (us * 1e-6) / 1e9
            res["by_rows"][str(r)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1),
                                      "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
            log("w8g32 %dx%d rows=%d (%d copies): %.2f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (
                n, k, r, copies, us, gbs, 100 * gbs / HBM_PEAK_GBS))
        out["%dx%d" % (n, k)] = res
        del cs
    return out


def time_norm(nv, torch, dev, reps):
    """nvfp4_residual_rmsnorm at the 27B model's hidden size (k = 5120): the
    average call at decode row counts (1 and 8: a few tens of KB, bound by
    latency) and GB/s at 4096 rows (reads residual and delta, writes
    residual_out and x: 8 bytes per element), cycling through >= 1 GiB of
    distinct buffers."""
    g = torch.Generator(device=dev).manual_seed(99)
    k = 5120
    w = torch.randn((k,), generator=g, device=dev).to(torch.bfloat16)
    out = {"k": k, "by_rows": {}}
    for rows in (1, 8, 4096):
        copies = max(1, -(-ROTATE_BYTES // (rows * k * 8)))
        copies = min(copies, 64)
        sets = []
        for _ in range(copies):
            r = torch.randn((rows, k), generator=g, device=dev).to(torch.bfloat16)
            h = torch.randn((rows, k), generator=g, device=dev).to(torch.bfloat16)
            sets.append((r, h, torch.empty_like(r), torch.empty_like(r)))
        us = time_rotating(torch, lambda i: nv.nvfp4_residual_rmsnorm(sets[i][0], sets[i][1], w,
                                                                      residual_out=sets[i][2], x=sets[i][3]),
                           copies, max(reps, 3 * copies))
        gbs = rows * k * 8 / (us * 1e-6) / 1e9
        out["by_rows"][str(rows)] = {"us": round(us, 2), "GB_per_s": round(gbs, 1), "copies": copies,
                                     "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        log("residual add + RMSNorm k=%d rows=%d (%d copies): %.2f us, %.1f GB/s" % (k, rows, copies, us, gbs))
        del sets
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

    if args.long_call_only:
        lbuf = torch.zeros(CEILING_BYTES, dtype=torch.uint8, device=dev)
        print(json.dumps({"long_call": time_long_call(nv, torch, dev, workloads, rows_list, args.steps, lbuf)}),
              flush=True)
        del lbuf
        torch.cuda.synchronize()
        return

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

    bufs = {r: {} for r in rows_list}
    seqs = {r: make_sequence(nv, torch, dev, workloads, mats, r, bufs[r]) for r in rows_list}
    ws = torch.zeros(max(s.workspace_bytes for s in seqs.values()), dtype=torch.uint8, device=dev)
    by_rows = {}
    parity = {}
    for r in rows_list:
        ms = time_rows(torch, seqs[r], ws, args.steps, args.warmup)
        if nv.wait_flag(ws):
            raise SystemExit("rows=%d: a wait between calls gave up (workspace wait flag set)" % r)
        if r in (1, 8) and not args.no_cpu_baseline:
            parity[str(r)] = parity_sample(nv, torch, mats, bufs[r], r)
            log("rows=%d: parity sample of layer %d: max err/sum|w*x| %.3g, max %d bf16 ulp, %d outputs"
                % (r, len(mats) - 1, parity[str(r)]["max_err_over_absdot"], parity[str(r)]["max_bf16_ulp"],
                   parity[str(r)]["outputs"]))
        pair_ms = None if args.step_only else time_pair(nv, torch, dev, mats, r, ws, max(2, args.steps // 10))
        gbs = step_bytes / (ms * 1e-3) / 1e9
        by_rows[str(r)] = {
            "ms_per_step": round(ms, 4),
            "launches_per_step": seqs[r].launches,
            "waits_per_step": seqs[r].waits,
            "GB_per_s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "gate_up_pair_us": None if pair_ms is None else round(pair_ms * 1e3, 3),
            "gate_up_pair_GB_per_s": None if pair_ms is None else round(pair_bytes / (pair_ms * 1e-3) / 1e9, 1),
        }
        log("rows=%d: %.4f ms/step in %d launches, %.1f GB/s (%.1f%% of 8 TB/s)%s"
            % (r, ms, seqs[r].launches, gbs, 100 * gbs / HBM_PEAK_GBS,
               "" if pair_ms is None else "; stand-alone gate/up pair %.2f us" % (pair_ms * 1e3)))

    # the same step with each layer's two residual add + RMSNorm calls inside
    # its launches (the activations of qkv and of the pair made by the step)
    with_norms = {}
    for r in [r for r in (1, 8) if r in rows_list and not args.step_only]:
        seq_n = make_sequence(nv, torch, dev, workloads, mats, r, norms=True)
        ms = time_rows(torch, seq_n, ws, max(5, args.steps // 2), min(args.warmup, 3))
        if nv.wait_flag(ws):
            raise SystemExit("rows=%d with norms: a wait between calls gave up" % r)
        base = by_rows[str(r)]["ms_per_step"]
        with_norms[str(r)] = {"ms_per_step": round(ms, 4), "launches_per_step": seq_n.launches,
                              "waits_per_step": seq_n.waits,
                              "calls_per_step": seq_n.n, "added_ms_vs_projections_only": round(ms - base, 4),
                              "added_us_per_norm": round((ms - base) * 1e3 / (2 * args.layers), 3)}
        log("rows=%d with %d fused residual add + RMSNorm calls: %.4f ms/step in %d launches (+%.3f us per norm)"
            % (r, 2 * args.layers, ms, seq_n.launches, (ms - base) * 1e3 / (2 * args.layers)))
        del seq_n

    wait_flag = nv.wait_flag(ws)
    if wait_flag:
        raise SystemExit("a wait between calls gave up (workspace wait flag set)")
    del seqs, bufs
    ceil_buf = None if args.step_only else torch.zeros(CEILING_BYTES, dtype=torch.uint8, device=dev)
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
        "traffic": load_traffic(rows_list[0]) if args.layers == 64 else None,
        "bytes_per_launch": round(launch_bytes),
        "avg_launch_us": round(launch_us, 2),
    }
    # the streaming-read ceiling of long reads (1 GiB per call, the step's
    # launch being longer), rotating through a 2 GiB buffer
    if not args.step_only:
        cbytes = min(int(launch_bytes) // 16 * 16, CEILING_BYTES // 2)
        cl = read_ceiling(nv, torch, dev, ceil_buf, cbytes, 20)
        ceiling_gbs = cbytes / (pctl(cl, 50) * 1e-6) / 1e9
        roofline["read_ceiling_GB_per_s"] = round(ceiling_gbs, 1)
        roofline["read_ceiling_bytes_per_call"] = cbytes
        roofline["frac_of_read_ceiling"] = round(achieved / ceiling_gbs, 4)
        log("read ceiling for %.2f GB reads: %.1f GB/s (%.1f%% of 8 TB/s); the step reaches %.1f%% of it"
            % (cbytes / 1e9, ceiling_gbs, 100 * ceiling_gbs / HBM_PEAK_GBS, 100 * achieved / ceiling_gbs))

    singles = None
    if args.layers == 64 and not args.step_only:
        singles = single_calls(nv, torch, dev, workloads, mats, ceil_buf)
        for key, v in singles.items():
            log("%s: median %.2f us (p10 %.2f, p90 %.2f), %.1f GB/s = %.1f%% of 8 TB/s; read ceiling %.2f us; "
                "floor at 75%%/70%%: %.2f us" % (key, v["median_us"], v["p10_us"], v["p90_us"], v["GB_per_s_median"],
                                                v["pct_hbm_peak_median"], v["read_ceiling_median_us"],
                                                v["derived_floor_us"]))

    long_call = None if args.step_only else time_long_call(
        nv, torch, dev, workloads, [r for r in (1, 8) if r in rows_list] or [rows_list[0]], 20, ceil_buf)

    dense = None
    skip_formats = args.no_dense or args.step_only
    if not skip_formats:
        dense = time_dense(nv, torch, dev, [r for r in (1, 8) if r in rows_list] or [rows_list[0]],
                           max(5, args.steps // 5))

    norm = None if skip_formats else time_norm(nv, torch, dev, max(10, args.steps // 2))
    # calls of 25-150 us: enough back-to-back calls that launch start-up is a small share
    mx = None if skip_formats else time_mx(nv, torch, dev, [r for r in (1, 8) if r in rows_list] or [rows_list[0]],
                                            max(50, args.steps))
    w8 = None if skip_formats else time_w8(nv, torch, dev, [r for r in (1, 8) if r in rows_list] or [rows_list[0]],
                                            max(50, args.steps))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on layer 0 ...")
        cpu = cpu_baseline(workloads, torch, dev, args.cpu_seconds)
        log("cpu baseline: %.3f GB/s on %d threads" % (cpu["value"], cpu["cores"]))

    del mats, ws
    gc.collect()
    torch.cuda.synchronize()

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
        "wait_timeouts": wait_flag,
        "parity_sample": parity or None,
        "single_calls": singles,
        "long_call": long_call,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_lm_head": dense,
        "residual_rmsnorm": norm,
        "step_with_norms": with_norms or None,
        "mxfp4": mx,
        "w8g32_f16s": w8,
    }
    print(json.dumps(line), flush=True)
    # end deterministically: nothing left on the device or in flight when the
    # interpreter (and any profiler attached to it) shuts down
    del ceil_buf
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    sys.stdout.flush()
    sys.stderr.flush()


if __name__ == "__main__":
    main()
