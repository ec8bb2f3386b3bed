"""Benchmark: mixed-bitrate quantized decode over a Llama-3-70B-shaped weight stack on one MI355X.

A step is one decode pass (M = 1 token by default) through all 80 decoder
blocks' seven linears (q, k, v, o, gate, up, down = 560 linears, ~22.9 GB of
2.55-bpw EXQ1 weights), each block's seven independent linears issued as one
exq plan launch.  Inputs are seeded synthetic tensors of the model's shapes
(no trained weights); they are resident in HBM before timing starts.

Prints one JSON line: whole-step HBM throughput (algorithmic bytes / step
time), ms/step, the decode kernel's roofline and the CPU oracle timed on a
bounded sample of the same workload.  Further legs:
  * step_back_to_back: the same step as 560 exq_gemm calls back to back
    (ungraphed and HIP-graph replayed), and as the launches a decoder
    block's data flow allows (q/k/v plan, o, fused gate/up, down);
  * prefill: the same seven 70B shapes at M = 2048 tokens (mixed 4.0 bpw
    from {3,4,5,6}) against the fp16 matrix-core peak, with the oracle timed
    on 64 seeded token rows and, as context, plain fp16 library GEMMs
    (torch.matmul) on the dequantized weights of the same shapes;
  * batched_decode_m16: the same stack at M = 16 rows;
  * single_layer: configurations 1 (4096 x 4096, 4-bit, M = 1) and 2
    (8192 x 8192, 2.55 bpw, M = 1/4/8/16), rotating over >= 1 GiB of copies;
  * stream_read, gated_gate_up, quantized_scales, autotune, allocator.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 5|3] [--m 1] [--no-prefill] [--no-batched]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "decode_plan_70b_m1_counters.json")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_plan_70b_m2048_counters.json")
# The prefill kernel and the plan builder that orders its tiles (the order sets its traffic).
PREFILL_SOURCES = ("exq_prefill.hip", "exq_device.hip", "exq_device_common.h", "exq_internal.h")


STREAM_READ_WGS = 8192   # workgroups of the streaming-read diagnostic (about 35 KB each per 286 MB)


def trimmed_mean(samples) -> float:
    """Mean of the samples that lie between the 5/16 and 11/16 quantiles
    (the middle three eighths of the sorted list)."""
    s = np.sort(np.asarray(samples, dtype=np.float64))
    n = len(s)
    lo, hi = (5 * n) // 16, max((11 * n + 15) // 16, (5 * n) // 16 + 1)
    return float(s[lo:hi].mean())


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_hash(files=("exq_device.hip", "exq_device_common.h", "exq_internal.h")) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixed_bitrate_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build_stack(exq, torch, specs, M, keep_first=0):
    """Generate, pack (host) and upload every linear; returns layers, xs, ys, bytes, kept W."""
    from synth import workloads
    layers, xs, ys, kept = [], [], [], []
    total = 0
    t0 = time.time()
    wbuf = None
    for i, spec in enumerate(specs):
        if wbuf is None or wbuf.size < spec.N * spec.K:
            wbuf = np.empty(spec.N * spec.K, dtype=np.float32)
        W = wbuf[: spec.N * spec.K].reshape(spec.N, spec.K)
        workloads.make_weight(spec, out=W)
        widths = workloads.make_widths(spec, W)
        q, s = exq.exq_pack(W, widths)
        if i < keep_first:
            kept.append((spec, W.copy(), widths))
        layers.append(exq.Layer(spec.K, spec.N, widths, q, s))
        xs.append(torch.from_numpy(workloads.make_x(spec, M)).cuda())
        ys.append(torch.empty((M, spec.N), dtype=torch.float16, device="cuda"))
        total += workloads.algorithmic_bytes(spec.K, spec.N, widths, M)
        if (i + 1) % 70 == 0 or i + 1 == len(specs):
            log("packed %d/%d linears (%.1f GB algorithmic) in %.0fs" % (i + 1, len(specs), total / 1e9, time.time() - t0))
    return layers, xs, ys, total, kept


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def event_timed(torch, stream, fn, reps, warmup=1):
    """Mean ms of `fn` over `reps` back-to-back runs between two events on `stream`."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graphed(torch, fn):
    """`fn`'s launches captured once as a HIP graph (returns the graph)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def omp_threads() -> int:
    import ctypes
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        return int(gomp.omp_get_max_threads())
    except OSError:
        return len(os.sched_getaffinity(0))


def cpu_baseline(kept, M, gpu_ys, min_seconds):
    """Time the CPU oracle (as it stands) on the kept linears: its own quantize+pack
    (untimed), then the timed path from packed storage -- bit-by-bit unpack,
    dequantize, fp64 matmul -- over every output column, repeated over the
    sample until at least `min_seconds` of timed work."""
    import oracle
    from synth import workloads
    prepared = []
    worst = 0.0
    for (spec, W, widths), y_gpu in zip(kept, gpu_ys):
        _, s_ref, q_ref = oracle.reference_layer(W, widths)
        prepared.append((spec, widths, s_ref, q_ref, workloads.make_x(spec, M), y_gpu))
    secs, nbytes, reps = 0.0, 0, 0
    while reps == 0 or secs < min_seconds:
        for spec, widths, s_ref, q_ref, x, y_gpu in prepared:
            cols = np.arange(spec.N, dtype=np.int64)
            t0 = time.perf_counter()
            y_ref, bnd = oracle.gemm_packed_cols(x, q_ref, s_ref, widths, spec.K, spec.N, cols)
            secs += time.perf_counter() - t0
            nbytes += workloads.algorithmic_bytes(spec.K, spec.N, widths, M)
            if reps == 0:
                _, w = oracle.within_tolerance(y_gpu.astype(np.float64), y_ref, bnd)
                worst = max(worst, w)
        reps += 1
    return secs, nbytes, worst, reps


def lp_lower_bound(err, size, budget, lo_opt):
    """Optimum of the linear relaxation of the multiple-choice knapsack (a
    lower bound on any allocation's error): each group's options above its
    minimum reduced to the lower convex hull of (bits, error), hull segments
    taken in order of error saved per bit, the last one fractionally."""
    WID = np.array([2, 3, 4, 5, 6, 8], dtype=np.float64)
    total = 0.0
    segs = []
    spent = 0.0
    for g in range(err.shape[0]):
        j0 = int(lo_opt[g])
        total += err[g, j0]
        spent += WID[j0] * size[g]
        hull = [j0]
        for j in range(j0 + 1, 6):
            if err[g, j] >= err[g, hull[-1]]:
                continue
            while len(hull) >= 2:
                a, b = hull[-2], hull[-1]
                if (err[g, a] - err[g, j]) / (WID[j] - WID[a]) >= (err[g, a] - err[g, b]) / (WID[b] - WID[a]):
                    hull.pop()
                else:
                    break
            hull.append(j)
        for a, b in zip(hull, hull[1:]):
            cost = (WID[b] - WID[a]) * size[g]
            segs.append(((err[g, a] - err[g, b]) / cost, cost, err[g, a] - err[g, b]))
    left = budget - spent
    for rate, cost, gain in sorted(segs, key=lambda s: -s[0]):
        if left <= 0:
            break
        take = min(1.0, left / cost)
        total -= take * gain
        left -= take * cost
    return total


def allocator_leg(exq, kept, nblk):
    """Host-side bit allocation (the offline step): measure block 0's seven
    linears (squared weight error at every width, exq_group_errors), then
    allocate widths over the whole stack at the seeded schedule's bit budget
    with the schedule's >= 6-bit groups kept (exq_allocate_widths; block 0's
    tables stand for every block)."""
    from synth import workloads
    if not kept:
        specs = workloads.linears(3)
        kept = []
        for spec in specs:
            W = workloads.make_weight(spec)
            kept.append((spec, W, workloads.make_widths(spec, W)))
    t0 = time.perf_counter()
    tables = [exq.exq_group_errors(W) for _, W, _ in kept]
    t_measure = time.perf_counter() - t0
    WID = np.array([2, 3, 4, 5, 6, 8])
    err = np.concatenate(tables * nblk)
    size = np.concatenate([np.full(t.shape[0], spec.N // 1024, dtype=np.int32) for (spec, _, _), t in zip(kept, tables)] * nblk)
    sched = np.concatenate([np.asarray(w, dtype=np.int64) for _, _, w in kept] * nblk)
    forced = np.where(sched >= 6, 6, 0).astype(np.uint8)
    budget = int((sched * size).sum())
    iters = 20 * err.shape[0]
    t0 = time.perf_counter()
    widths, total = exq.exq_allocate_widths(err, size, budget, forced, seed=1, iterations=iters)
    t_alloc = time.perf_counter() - t0
    sched_err = float(err[np.arange(err.shape[0]), np.searchsorted(WID, sched)].sum())
    bound = lp_lower_bound(err, size, budget, np.where(forced >= 6, 4, 0))
    bits = int((widths.astype(np.int64) * size).sum())
    log("allocator: measure %.2f s, allocate %d groups %.2f s, error %.4g vs schedule %.4g" % (
        t_measure, err.shape[0], t_alloc, total, sched_err))
    return {"measure_s_block0": round(t_measure, 3), "allocate_s_stack": round(t_alloc, 3), "groups": int(err.shape[0]),
            "iterations": iters, "cores": omp_threads(),
            "bpw_allocated": round(bits / float(size.sum()), 4),
            "error_vs_seeded_schedule": round(total / sched_err, 4),
            "error_vs_lp_lower_bound": round(total / bound, 6),
            "workload": "squared weight error of block 0's 7 linears at 2..8 bits; widths for the %d-block stack at "
                        "the seeded schedule's budget (2.55 bpw per linear), its >= 6-bit groups kept" % nblk}


def qs_leg(exq, torch, M, steps, stream, fp16_plans, nblk=8, rounds=3):
    """Decode with quantized group scales (4-bit codes + a column reference):
    `nblk` 70B-shaped blocks (2.2 GB, well above the Infinity Cache) packed with
    exq_pack_qs, one plan launch per block, rotating over the blocks.  The same
    number of fp16-scale block plans of the same shapes (`fp16_plans`) is timed
    in alternation with them, `rounds` times each, so that both figures come
    from the same stretch of the run (clock and cache state alike)."""
    from synth import BLOCK_SHAPES, workloads
    specs = workloads.linears(5)[: nblk * len(BLOCK_SHAPES)]
    layers, xs, ys, nbytes = [], [], [], 0
    for spec in specs:
        W = workloads.make_weight(spec)
        widths = workloads.make_widths(spec, W)
        q, qsc, ref = exq.exq_pack_qs(W, widths)
        layers.append(exq.Layer(spec.K, spec.N, widths, q, qsc, ref=ref))
        xs.append(torch.from_numpy(workloads.make_x(spec, M)).cuda())
        ys.append(torch.empty((M, spec.N), dtype=torch.float16, device="cuda"))
        G = spec.K // 128
        nbytes += q.size + qsc.size + 2 * spec.N + 5 * G + 2 * M * spec.K + 2 * M * spec.N
    plans = [exq.Plan(layers[b * 7:(b + 1) * 7], xs[b * 7:(b + 1) * 7], ys[b * 7:(b + 1) * 7], M) for b in range(nblk)]
    reps = max(steps, 40)

    def timed(ps):
        for _ in range(10):
            for p in ps:
                p.run(stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for p in ps:
                p.run(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(ps))

    qs_us, fp_us = [], []
    for _ in range(rounds):
        qs_us.append(timed(plans))
        fp_us.append(timed(fp16_plans[:nblk]))
    us_block, fp_block = float(np.median(qs_us)), float(np.median(fp_us))
    for p in plans:
        p.close()
    for l in layers:
        l.close()
    per_block = nbytes / nblk
    log("quantized scales: %.1f us per block (fp16 scales, same shapes, alternated: %.1f us), %.0f B per block" % (
        us_block, fp_block, per_block))
    return {"workload": "%d llama3-70b-shaped blocks, 2.55 bpw, 4-bit group scale codes, M=%d, one plan per block" % (nblk, M),
            "us_per_block": round(us_block, 2), "bytes_per_block": int(per_block),
            "GB/s": round(per_block / (us_block * 1e-6) / 1e9, 1),
            "fp16_scales_us_per_block_same_blocks": round(fp_block, 2),
            "timing": "median over %d alternated rounds of %d steps over the %d blocks, each after 10 warmup steps" % (
                rounds, reps, nblk),
            "ms_per_step_80_blocks_equivalent": round(us_block * 80 / 1e3, 4)}


def autotune_leg(exq, torch, layers, stream, Ms=(1, 4, 16, 32)):
    """exq_autotune on block 0's seven linears at several row counts (20 warmup
    and 200 timed runs per candidate, trimmed mean of the 5/16-11/16
    quantiles); the choices are reset afterwards."""
    from synth import BLOCK_SHAPES
    names = ["decode16", "decode64", "prefill"]
    out = {}
    for M in Ms:
        rows = []
        for (name, K, N), lay in zip(BLOCK_SHAPES, layers):
            x = torch.randn((M, K), device="cuda").half()
            y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            choice, times = exq.exq_autotune(x.data_ptr(), M, lay.handle, y.data_ptr(), stream, 20, 200)
            m = min(M, 16)   # exq_gemm's default: decode slices of 16 rows, this tile rule
            default = 2 if (m > 4 or N // 64 >= 256 or (m >= 4 and N // 64 >= 128)) else 1
            rows.append({"linear": name, "choice": names[choice - 1], "us": round(times[choice - 1], 2),
                         "default_us": round(times[default - 1], 2),
                         "candidates_us": [round(t, 2) for t in times]})
            exq.exq_set_variant(lay.handle, M, 0)
        out["M=%d" % M] = rows
        log("autotune M=%d: %s" % (M, ", ".join("%s %s %.1f/%.1f us" % (r["linear"], r["choice"], r["us"], r["default_us"])
                                                for r in rows)))
    return out


def batched_decode_leg(exq, torch, specs, layers, nblk, M, steps, stream):
    """The same stack streamed per step at M rows (the batched-decode shape):
    one decode plan per block, as in the headline step, on fresh x and y."""
    from synth import workloads
    xs = [torch.from_numpy(workloads.make_x(sp, M)).cuda() for sp in specs]
    ys = [torch.empty((M, sp.N), dtype=torch.float16, device="cuda") for sp in specs]
    per = len(specs) // nblk
    plans = [exq.Plan(layers[b * per:(b + 1) * per], xs[b * per:(b + 1) * per], ys[b * per:(b + 1) * per], M)
             for b in range(nblk)]
    nbytes = sum(workloads.algorithmic_bytes(sp.K, sp.N, l.widths, M) for sp, l in zip(specs, layers))

    def step():
        for p in plans:
            p.run(stream)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for p in plans:
        p.close()
    del xs, ys
    torch.cuda.empty_cache()
    log("M=%d stack step %.3f ms, %.1f GB/s" % (M, ms, nbytes / (ms * 1e-3) / 1e9))
    return {"workload": "the same %d-block stack at M=%d, one decode plan per block" % (nblk, M), "M": M,
            "ms_per_step": round(ms, 4), "bytes_per_step": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2), "steps": steps}


def gated_leg(exq, torch, layers, xs, M, nblk, steps, stream):
    """The 80 gate/up pairs of the stack: h = SiLU(x Wg^T) * (x Wu^T) per block
    as one exq_gemm_gated launch, against a two-linear plan plus torch's SiLU
    and multiply (three launches and two fp16 intermediates)."""
    from synth import BLOCK_SHAPES
    names = [s[0] for s in BLOCK_SHAPES]
    ig, iu = names.index("gate"), names.index("up")
    pairs = [(layers[b * len(names) + ig], layers[b * len(names) + iu], xs[b * len(names) + ig]) for b in range(nblk)]
    N = pairs[0][0].N
    hs = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in range(nblk)]
    gs = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in range(nblk)]
    us = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in range(nblk)]
    plans = [exq.Plan([g, u], [x, x], [gs[b], us[b]], M) for b, (g, u, x) in enumerate(pairs)]

    def fused():
        for (g, u, x), h in zip(pairs, hs):
            exq.exq_gemm_gated(x.data_ptr(), M, g.handle, u.handle, h.data_ptr(), stream)

    def separate():
        for b, p in enumerate(plans):
            p.run(stream)
            torch.mul(torch.nn.functional.silu(gs[b]), us[b], out=hs[b])

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_fused, ms_sep = timed(fused), timed(separate)
    for p in plans:
        p.close()
    nbytes = 0
    for g, u, x in pairs:
        for l in (g, u):
            nbytes += int(l.qweight.numel()) + int(l.scales.numel()) * 2 + 5 * (l.K // 128)
        nbytes += 2 * M * g.K + 2 * M * N
    log("gated gate/up: fused %.3f ms, plan + torch SiLU*mul %.3f ms per step" % (ms_fused, ms_sep))
    return {"workload": "the %d gate/up pairs (8192 -> 28672, 2.55 bpw) of the stack, M=%d" % (nblk, M),
            "ms_per_step_fused": round(ms_fused, 4), "GB/s_fused": round(nbytes / (ms_fused * 1e-3) / 1e9, 1),
            "ms_per_step_plan_plus_torch_silu_mul": round(ms_sep, 4),
            "bytes_per_step": nbytes}


def prefill_oracle_subset(kept, xs, ys, rows_n, seed):
    """The oracle on `rows_n` seeded token rows of every linear, every output
    column (its own packed layer; unpack + dequant + fp64 matmul timed), and
    the worst error / tolerance of the GPU's rows."""
    import oracle
    rng = np.random.default_rng(seed)
    secs, flops, worst = 0.0, 0, 0.0
    for (spec, W, widths), x, y in zip(kept, xs, ys):
        _, s_ref, q_ref = oracle.reference_layer(W, widths)
        rows = np.sort(rng.choice(x.shape[0], size=rows_n, replace=False))
        xr = x[rows].cpu().numpy()
        cols = np.arange(spec.N, dtype=np.int64)
        t0 = time.perf_counter()
        y_ref, bnd = oracle.gemm_packed_cols(xr, q_ref, s_ref, widths, spec.K, spec.N, cols)
        secs += time.perf_counter() - t0
        flops += 2 * rows_n * spec.K * spec.N
        _, w = oracle.within_tolerance(y[rows].cpu().numpy().astype(np.float64), y_ref, bnd)
        worst = max(worst, w)
    return secs, flops, worst


def prefill_leg(exq, torch, steps, warmup, oracle_rows=64, dense_ref=True):
    """The seven 70B-shaped linears at M = 2048 (mixed 4.0 bpw) as one prefill
    plan launch per step; step time, the launch's own duration, and the same
    step as seven separate exq_gemm calls for reference.  The oracle is timed
    on a seeded subset of token rows (every column of every linear)."""
    from synth import workloads
    M = workloads.M_VALUES[4][0]
    specs = workloads.linears(4)
    layers, xs, ys, _, kept = build_stack(exq, torch, specs, M, keep_first=len(specs) if oracle_rows else 0)
    flops = sum(2 * M * sp.K * sp.N for sp in specs)
    stream = torch.cuda.current_stream()
    plan = exq.Plan(layers, xs, ys, M)

    def timed(fn, reps):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    ms_step = timed(lambda: plan.run(stream), steps)
    kernel_ms = ms_step   # one plan launch per step, back to back: the timed region's average launch

    def calls():
        for l, x, y in zip(layers, xs, ys):
            exq.exq_gemm(x.data_ptr(), M, l.handle, y.data_ptr(), stream)
    ms_calls = timed(calls, max(3, steps // 2))

    # Context, not the path: the same seven products as plain fp16 library
    # GEMMs (torch.matmul, which calls hipBLASLt / rocBLAS) on the dequantized
    # weights W_hat [K][N], a practical matrix-core ceiling for these shapes.
    dense = None
    if dense_ref:
        ws = [l.dequant(stream) for l in layers]
        dys = [torch.empty_like(y) for y in ys]

        def dense_step():
            for x, w, y in zip(xs, ws, dys):
                torch.matmul(x, w, out=y)
        ms_dense = timed(dense_step, max(3, steps // 2))
        dense = {"ms_per_step": round(ms_dense, 4), "TFLOP/s": round(flops / (ms_dense * 1e-3) / 1e12, 2),
                 "pct_of_peak": round(100 * flops / (ms_dense * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 2),
                 "kernel": "torch.matmul (hipBLASLt / rocBLAS) fp16 x fp16 -> fp16, 7 calls on the dequantized weights",
                 "weight_bytes_fp16": int(sum(w.numel() * 2 for w in ws))}
        del ws, dys
        torch.cuda.empty_cache()
        log("dense fp16 library GEMMs on W_hat: %.3f ms per step, %.1f TFLOP/s" % (ms_dense, dense["TFLOP/s"]))
    cpu = None
    if oracle_rows:
        plan.run(stream)
        torch.cuda.synchronize()
        log("timing the oracle on %d rows of each prefill linear" % oracle_rows)
        secs, cflops, worst = prefill_oracle_subset(kept, xs, ys, oracle_rows, 4242)
        cpu = {"value": round(cflops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": omp_threads(), "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": "%d seeded token rows of each of the 7 linears (of %d), every output column: bit-by-bit "
                         "unpack + dequant + fp64 matmul from the oracle's own packed layer; %.1f s for %.3g flop; "
                         "worst GPU error / tolerance on those rows %.3f" % (oracle_rows, M, secs, cflops, worst)}
    plan.close()
    for l in layers:
        l.close()
    tflops = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(PREFILL_COUNTERS):
        with open(PREFILL_COUNTERS) as f:
            prof = json.load(f)
        if prof.get("kernel_source_hash") == kernel_source_hash(PREFILL_SOURCES):
            traffic = prof.get("hbm_bytes_per_launch")
    log("prefill step %.3f ms, %.1f TFLOP/s; launch %.3f ms (%.1f TFLOP/s); 7 calls %.3f ms" % (
        ms_step, tflops, kernel_ms, achieved, ms_calls))
    return {
        "workload": "llama3-70b-shaped block (7 linears), mixed 4.0 bpw {3,4,5,6}, M=%d tokens" % M,
        "metric": "prefill TFLOP/s (one plan launch per step)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_separate_calls": round(ms_calls, 4),
        "dense_fp16_library_gemm": dense,
        "steps": steps,
        "warmup": warmup,
        "flops_per_step": flops,
        "cpu_baseline": cpu,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "prefill_plan_kernel (one launch = the block's 7 linears)",
            "flops_per_launch": flops,
            "avg_launch_ms": round(kernel_ms, 4),
        },
    }


def back_to_back_leg(exq, torch, specs, layers, xs, ys, nblk, M, steps, stream, step_bytes):
    """The step as a sequence of launches, every linear its own call:
      * per_linear: the 560 (or 7) linears as exq_gemm calls back to back on
        one stream, ungraphed and captured once as a HIP graph;
      * dependent: the launches a decoder block's data flow allows -- q, k
        and v as one plan on one shared x, then o, then gate and up fused
        with their SiLU product (exq_gemm_gated), then down reading that
        product -- ungraphed and graphed.  o's input (the attention output)
        and gate/up's input (the next normalised hidden state) come from
        outside this library and are fixed synthetic buffers.
    Bytes per step are the headline's (the 560 linears' algorithmic bytes)."""
    from synth import BLOCK_SHAPES
    names = [b[0] for b in BLOCK_SHAPES]
    per = len(names)
    iq, ik, iv, io, ig, iu, idn = (names.index(n) for n in ("q", "k", "v", "o", "gate", "up", "down"))

    def calls(st):
        for l, x, y in zip(layers, xs, ys):
            exq.exq_gemm(x.data_ptr(), M, l.handle, y.data_ptr(), st)

    ms_calls = event_timed(torch, stream, lambda: calls(stream), steps)
    g = graphed(torch, calls)
    ms_calls_g = event_timed(torch, stream, g.replay, steps)
    del g

    blocks = []
    for b in range(nblk):
        L = layers[b * per:(b + 1) * per]
        X = xs[b * per:(b + 1) * per]
        # Own outputs: k, v and down here read other inputs than the stack's own
        # x buffers, and the stack's outputs are checked against the oracle later.
        Y = [torch.empty_like(y) for y in ys[b * per:(b + 1) * per]]
        h = torch.empty((M, L[ig].N), dtype=torch.float16, device="cuda")
        qkv = exq.Plan([L[iq], L[ik], L[iv]], [X[iq], X[iq], X[iq]], [Y[iq], Y[ik], Y[iv]], M)
        blocks.append((qkv, L, X, Y, h))

    def dependent(st):
        for qkv, L, X, Y, h in blocks:
            qkv.run(st)
            exq.exq_gemm(X[io].data_ptr(), M, L[io].handle, Y[io].data_ptr(), st)
            exq.exq_gemm_gated(X[ig].data_ptr(), M, L[ig].handle, L[iu].handle, h.data_ptr(), st)
            exq.exq_gemm(h.data_ptr(), M, L[idn].handle, Y[idn].data_ptr(), st)

    ms_dep = event_timed(torch, stream, lambda: dependent(stream), steps)
    g = graphed(torch, dependent)
    ms_dep_g = event_timed(torch, stream, g.replay, steps)
    del g
    for qkv, *_ in blocks:
        qkv.close()
    del blocks
    gbs = lambda ms: round(step_bytes / (ms * 1e-3) / 1e9, 1)
    log("back to back: %d exq_gemm calls %.3f ms (graphed %.3f); dependent schedule %.3f ms (graphed %.3f)" % (
        len(layers), ms_calls, ms_calls_g, ms_dep, ms_dep_g))
    return {
        "per_linear": {"launches_per_step": len(layers), "ms_per_step": round(ms_calls, 4), "GB/s": gbs(ms_calls),
                       "ms_per_step_graphed": round(ms_calls_g, 4), "GB/s_graphed": gbs(ms_calls_g),
                       "us_per_block": round(ms_calls * 1e3 / nblk, 2),
                       "us_per_block_graphed": round(ms_calls_g * 1e3 / nblk, 2)},
        "dependent": {"launches_per_step": 4 * nblk, "ms_per_step": round(ms_dep, 4), "GB/s": gbs(ms_dep),
                      "ms_per_step_graphed": round(ms_dep_g, 4), "GB/s_graphed": gbs(ms_dep_g),
                      "us_per_block": round(ms_dep * 1e3 / nblk, 2),
                      "us_per_block_graphed": round(ms_dep_g * 1e3 / nblk, 2),
                      "schedule": "per block: plan(q,k,v on one x) -> exq_gemm(o) -> exq_gemm_gated(gate,up) -> "
                                  "exq_gemm(down on the gated output)"},
        "steps": steps,
    }


def single_layer_leg(exq, torch, config, stream, reps=200, warmup=20, min_bytes=1 << 30):
    """Configuration 1 or 2: one layer, exq_gemm at each M the configuration
    names, rotating over distinct device copies of the packed layer totalling
    at least 1 GiB (four times the 256 MB Infinity Cache), so every call reads
    its weights from HBM.  `warmup` untimed and `reps` timed calls back to
    back: the mean from two events around them, and the median and trimmed
    mean (5/16-11/16 quantiles) of per-call event pairs in a second pass
    (each pair adds its own few microseconds)."""
    from synth import workloads
    spec = workloads.linears(config)[0]
    W = workloads.make_weight(spec)
    widths = workloads.make_widths(spec, W)
    q, sc = exq.exq_pack(W, widths)
    per_copy = workloads.algorithmic_bytes(spec.K, spec.N, widths, 1)
    copies = -(-min_bytes // per_copy)
    layers = [exq.Layer(spec.K, spec.N, widths, q, sc) for _ in range(copies)]
    out = {"workload": "%d -> %d, %s, %d rotating copies (%.2f GB)" % (
        spec.K, spec.N, "uniform 4-bit" if spec.kind == "u4" else "mixed 2.55 bpw", copies,
        copies * per_copy / 1e9), "rows": []}
    for M in workloads.M_VALUES[config]:
        x = torch.from_numpy(workloads.make_x(spec, M)).cuda()
        y = torch.empty((M, spec.N), dtype=torch.float16, device="cuda")
        it = [0]

        def call():
            l = layers[it[0] % copies]
            it[0] += 1
            exq.exq_gemm(x.data_ptr(), M, l.handle, y.data_ptr(), stream)

        ms = event_timed(torch, stream, call, reps, warmup)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        samples = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
        nbytes = workloads.algorithmic_bytes(spec.K, spec.N, widths, M)
        out["rows"].append({"M": M, "us_per_call": round(ms * 1e3, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                            "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                            "bytes_per_call": nbytes,
                            "median_us_event_pairs": round(float(np.median(samples)), 3),
                            "trimmed_mean_us_event_pairs": round(trimmed_mean(samples), 3)})
    for l in layers:
        l.close()
    log("config %d: %s" % (config, ", ".join("M=%d %.2f us %.0f GB/s" % (r["M"], r["us_per_call"], r["GB/s"])
                                             for r in out["rows"])))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=5, choices=(3, 5))
    ap.add_argument("--m", type=int, default=1)
    ap.add_argument("--blocks", type=int, default=None, help="limit the number of 70B blocks (config 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=1, help="blocks of the workload the oracle is timed on")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="minimum timed oracle work (the sample is repeated)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M = 2048 prefill leg")
    ap.add_argument("--no-batched", action="store_true", help="skip the M = 16 pass over the stack")
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--prefill-warmup", type=int, default=10)
    ap.add_argument("--prefill-oracle-rows", type=int, default=64, help="token rows the oracle is timed on (0: none)")
    ap.add_argument("--no-back-to-back", action="store_true", help="skip the per-linear and dependent schedules")
    ap.add_argument("--no-single", action="store_true", help="skip the single-layer rows (configurations 1 and 2)")
    ap.add_argument("--no-stream-read", action="store_true", help="skip the plain streaming-read ceiling")
    ap.add_argument("--no-gated", action="store_true", help="skip the fused gate/up (SiLU) leg")
    ap.add_argument("--no-allocator", action="store_true", help="skip the host bit-allocation leg")
    ap.add_argument("--no-autotune", action="store_true", help="skip the per-shape kernel-choice leg")
    ap.add_argument("--no-qs", action="store_true", help="skip the quantized-scale decode leg")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense fp16 library GEMM context of the prefill leg")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="run a plain device copy of this size (for counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import mixed_bitrate_quantized_amd as exq
    from synth import workloads, BLOCK_SHAPES

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30)) // 2
        a = torch.empty(n, dtype=torch.float16, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copied %d bytes three times" % (2 * n))
        return

    M = args.m
    specs = workloads.linears(args.config)
    if args.blocks is not None:
        specs = specs[: args.blocks * len(BLOCK_SHAPES)]
    nblk = len(specs) // len(BLOCK_SHAPES)
    keep = 0 if args.no_cpu_baseline else args.cpu_blocks * len(BLOCK_SHAPES)
    layers, xs, ys, step_bytes, kept = build_stack(exq, torch, specs, M, keep_first=keep)
    plans = []
    for b in range(nblk):
        sl = slice(b * len(BLOCK_SHAPES), (b + 1) * len(BLOCK_SHAPES))
        plans.append(exq.Plan(layers[sl], xs[sl], ys[sl], M))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step():
        for p in plans:
            p.run(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly `steps` steps between two events on the launch stream.
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_begin.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_begin.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # The decode kernel's average launch duration over the timed region: its
    # launches run back to back on the stream (a kernel trace shows each one
    # starting as the previous ends), so the region's time over its launch
    # count is that average.  (An event pair around every launch would add
    # its own gap, about 5-10 us, to every sample.)
    kernel_ms = ms_total / (args.steps * nblk)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    bytes_per_launch = step_bytes / nblk
    achieved = bytes_per_launch / (kernel_ms * 1e-3) / 1e9
    log("step %.3f ms, %.1f GB/s; decode launch %.1f us (%.1f GB/s)" % (ms_step, gbs, kernel_ms * 1e3, achieved))

    # Per-step durations (an event pair around every step, a third pass) for
    # the median and the trimmed mean of the 5/16-11/16 quantiles.
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in step_ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in step_ev])
    step_stats = {"median_ms": round(float(np.median(per_step)), 4),
                  "trimmed_mean_ms": round(trimmed_mean(per_step), 4),
                  "min_ms": round(float(per_step.min()), 4), "max_ms": round(float(per_step.max()), 4),
                  "trimmed_mean": "mean of the per-step times between the 5/16 and 11/16 quantiles"}

    # The same step captured once as a HIP graph and replayed.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for p in plans:
            p.run(cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    ms_step_graphed = g0.elapsed_time(g1) / args.steps
    del graph

    # Diagnostic ceiling: a plain streaming read of the same bytes, one launch
    # per block (cold: 16 windows rotate through HBM), same step structure.
    read = None
    if not args.no_stream_read:
        win = (int(bytes_per_launch) // 16) * 16
        copies = 16
        rbuf = torch.empty(copies * win // 4, dtype=torch.int32, device="cuda").fill_(1)
        sink = torch.zeros(STREAM_READ_WGS, dtype=torch.int32, device="cuda")
        base = rbuf.data_ptr()

        def read_step(s):
            for b in range(nblk):
                exq.exq_stream_read(base + ((s * nblk + b) % copies) * win, win, sink.data_ptr(), STREAM_READ_WGS,
                                    stream)

        for s in range(2):
            read_step(s)
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for s in range(args.steps):
            read_step(s)
        r1.record(stream)
        torch.cuda.synchronize()
        read_ms = r0.elapsed_time(r1) / args.steps
        read_gbs = win * nblk / (read_ms * 1e-3) / 1e9
        read = {"ms_per_step": round(read_ms, 4), "GB/s": round(read_gbs, 1),
                "decode_pct_of_stream_read": round(100 * gbs / read_gbs, 1),
                "kernel": "stream_read_kernel, %d workgroups per launch, %d B per launch" % (STREAM_READ_WGS, win)}
        del rbuf, sink
        torch.cuda.empty_cache()
    log("graphed step %.3f ms; stream read %s" % (ms_step_graphed, read))

    gated = None
    if not args.no_gated and args.config == 5:
        gated = gated_leg(exq, torch, layers, xs, M, nblk, args.steps, stream)

    batched = None
    if not args.no_batched and args.config == 5 and M == 1:
        batched = batched_decode_leg(exq, torch, specs, layers, nblk, 16, max(5, args.steps // 5), stream)

    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        with open(PROFILE_COUNTERS) as f:
            prof = json.load(f)
        if prof.get("kernel_source_hash") == kernel_source_hash() and prof.get("config") == args.config and prof.get("m") == M:
            traffic = prof.get("hbm_bytes_per_launch")

    b2b = None
    if not args.no_back_to_back:
        b2b = back_to_back_leg(exq, torch, specs, layers, xs, ys, nblk, M, args.steps, stream, step_bytes)

    cpu = None
    if kept:
        log("timing the CPU oracle on %d linears" % len(kept))
        gpu_ys = [ys[i].cpu().numpy() for i in range(len(kept))]
        secs, cbytes, worst, reps = cpu_baseline(kept, M, gpu_ys, args.cpu_seconds)
        cpu = {
            "value": round(cbytes / secs / 1e9, 4),
            "unit": "GB/s",
            "cores": omp_threads(),
            "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d linears (block%s 0..%d of the same stack) at M=%d, every output column, %d passes: "
                      "bit-by-bit unpack + dequant + fp64 matmul from the oracle's own packed layer; %.1f s for "
                      "%.2f GB; worst GPU error / tolerance on the sample %.3f" % (
                          len(kept), "s" if args.cpu_blocks > 1 else "", args.cpu_blocks - 1, M, reps, secs,
                          cbytes / 1e9, worst),
        }

    qsres = None
    if not args.no_qs and args.config == 5:
        qsres = qs_leg(exq, torch, M, args.steps, stream, plans, nblk=min(8, len(plans)))
        qsres["fp16_scales_us_per_block_whole_stack"] = round(ms_step * 1e3 / nblk, 2)

    tune = None
    if not args.no_autotune:
        tune = autotune_leg(exq, torch, layers[: len(BLOCK_SHAPES)], stream)

    alloc = None
    if not args.no_allocator and args.config == 5:
        alloc = allocator_leg(exq, kept if len(kept) == len(BLOCK_SHAPES) else None, nblk)

    prefill = None
    if not args.no_prefill:
        for p in plans:
            p.close()
        for l in layers:
            l.close()
        del layers, xs, ys, plans
        torch.cuda.empty_cache()
        prefill = prefill_leg(exq, torch, args.prefill_steps, args.prefill_warmup, args.prefill_oracle_rows,
                              dense_ref=not args.no_dense)

    single = None
    if not args.no_single:
        torch.cuda.empty_cache()
        single = {"config1": single_layer_leg(exq, torch, 1, torch.cuda.current_stream()),
                  "config2": single_layer_leg(exq, torch, 2, torch.cuda.current_stream())}

    out = {
        "metric": "quant GEMV eff. HBM GB/s (% peak) + ms/step, 70B-shaped 2.55bpw M=" + str(M),
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in, fp32 accumulate, EXQ1 2-8 bit codes",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) fp16 activations)",
        "config": {
            "workload": ("llama3-70b-shaped decoder stack: %d blocks x 7 linears, mixed 2.55 bpw, M=%d" % (nblk, M))
            if args.config == 5 else "one llama3-70b-shaped block (7 linears), mixed 2.55 bpw, M=%d" % M,
            "linears": len(specs),
            "bytes_per_step": step_bytes,
            "launches_per_step": nblk,
            "step": "one decode plan launch per block: the block's 7 linears, each on its own synthetic input, in "
                    "one kernel (back-to-back and data-flow schedules in step_back_to_back)",
            "parallelism": "1 GPU",
        },
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "decode_plan_kernel (one launch = one block's 7 linears)",
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": round(kernel_ms * 1e3, 3),
        },
        "ms_per_step_graphed": round(ms_step_graphed, 4),
        "step_stats": step_stats,
        "step_back_to_back": b2b,
        "single_layer": single,
        "stream_read": read,
        "gated_gate_up": gated,
        "batched_decode_m16": batched,
        "allocator": alloc,
        "autotune": tune,
        "quantized_scales": qsres,
        "cpu_baseline": cpu,
        "prefill": prefill,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
