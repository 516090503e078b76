"""Benchmark of the microscaled hot path on one MI355X.

One step is the whole path on one batch of synthetic input, back to back on one stream:
act_quant of bf16 activations x [4096, 2048] (N(0,1) with 1% of entries x100) into E4M3 codes +
E8M0 scales, then the FP8 x MXFP4 GEMM against E2M1 weights [7168, 2048] (per-32 E8M0 scales
118..136) with a fused bf16 bias, bf16 out [4096, 7168].

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all]
    python bench.py --summarize STATS_DIR FETCH_DIR WRITE_DIR   (CPU only; writes profiles/)
    python bench.py --summarize-busy BUSY_DIR                   (CPU only; writes profiles/)

Prints one JSON line.  `value` is the GEMM's 2*M*N*K flops divided by the time of a whole step
(act_quant included), in TFLOP/s, over the caller's --warmup and --steps.

Every kernel figure besides `value` comes from `gemm_leg`-style timing that does not depend on
those flags: launches back to back for at least 100 ms of wall-clock time first (past the clock
drop that sustained load brings), then 12 groups of 10 back-to-back launches, one pair of HIP
events per group on the stream the launches go to; the figure is the median of the 12 group
means (120 launches).  `roofline` is the dominant kernel (the 4096x7168x2048 GEMM) timed that
way, against the dense FP8 MFMA peak.  `gemm_8192cubed` and `gemm_batched_8x1024x2048x2048` are
the two large FP8 x FP8 configurations, each with its own roofline block.  Each of the three large GEMM
blocks also carries `cold_ms`: the median of 10 single launches, each after 512 MB were written to
evict the caches (taken before the leg's timed launches).  `latency` holds the
small configurations (16x256x512, 1024^3 + bias and the three skinny A4W4 shapes): the same
median, `graph_ms` (20 launches captured in one HIP graph, replayed; launch overhead amortized)
and `cold_ms` (median of single launches, each after 512 MB were written to evict the caches).
Each of the three large GEMM blocks carries `vendor_bf16`: the vendor library's plain bf16 GEMM
(torch.matmul) on the same shape, timed in alternation with ours (same clock and temperature),
as context: what the bf16 MFMA reaches on this GPU without decodes or scales.  The next-layer
leg times its fused and unfused variants in alternation too.  `act_quant` reports the standalone
producer on [16384, 7168] against HBM bandwidth,
`act_quant_fp4` the MXFP4 producer on the same input.  `cpu_baseline` times the oracle on a
bounded sample of the same workload on the host.  Each roofline block names the kernel and grid
of its dispatches and how many of them it timed (`trace`), so that a kernel trace of the same
command can be matched against it (--summarize).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
METRIC = "block-scaled GEMM TFLOP/s (% MFMA peak) + act_quant GB/s (% HBM peak)"
ACT_QUANT_BYTES_PER_ELEM = 2 + 1 + 1 / 32      # bf16 in, E4M3 code out, one scale byte per 32
ACT_QUANT_FP4_BYTES_PER_ELEM = 2 + 0.5 + 1 / 32   # bf16 in, half a byte of E2M1 out, scale per 32
SETTLE_MS = 100.0             # wall-clock warm-up of every timed kernel leg
GROUPS, PER_GROUP = 12, 10    # timed launches: GROUPS groups of PER_GROUP back-to-back launches


GEMM_SOURCES = ["block_scaled_precision_act_amd/csrc/gemm_bf16.hip",
                "block_scaled_precision_act_amd/csrc/gemm_mx.hip",
                "block_scaled_precision_act_amd/csrc/gemm_common.h",
                "block_scaled_precision_act_amd/csrc/mx_internal.h",
                "block_scaled_precision_act_amd/csrc/mx_epilogue.h",
                "block_scaled_precision_act_amd/csrc/mx_quant.h"]
FP4_SOURCES = ["block_scaled_precision_act_amd/csrc/gemm_fp4.hip",
               "block_scaled_precision_act_amd/csrc/mx_internal.h",
               "block_scaled_precision_act_amd/csrc/mx_epilogue.h",
               "block_scaled_precision_act_amd/csrc/mx_quant.h"]
ACT_QUANT_SOURCES = ["block_scaled_precision_act_amd/csrc/act_quant.hip",
                     "block_scaled_precision_act_amd/csrc/mx_philox.h",
                     "block_scaled_precision_act_amd/csrc/mx_quant.h"]
# act_quant_kernel<chunks per lane, output format, stochastic>: format 0 is E4M3, 4 packed E2M1
AQ_E4M3_KERNEL = r"act_quant_kernel<\d+, 0, false>"
AQ_E2M1_KERNEL = r"act_quant_kernel<\d+, 4, false>"
# gemm_mx_kernel<A format, B format, bias, quantized output, epilogue, split-K, tile width>
# (256 x 256 or 256 x 224 tiles, 256 threads) and gemm_bf16_kernel<same first six, BM, BN, WM, WN>
# (smaller tiles): format 0 is E4M3, 4 packed E2M1.  4096 x 7168 takes 256 x 224 tiles (512
# tiles: two full waves of 256 CUs), the others 256 x 256.
GEMM_FP8_FP4_KERNEL = r"gemm_mx_kernel<0, 4, true, false, 0, false, 224>"
GEMM_FP8_FP4_QUANT_KERNEL = r"gemm_mx_kernel<0, 4, true, true, 0, false, 224>"
GEMM_FP8_FP4_128_KERNEL = r"gemm_bf16_kernel<0, 4, true, false, 0, false, 128, 128,"
GEMM_FP8_FP4_SPLITK_KERNEL = r"gemm_mx_kernel<0, 4, true, false, 0, true, 256>"
GEMM_FP8_FP8_KERNEL = r"gemm_mx_kernel<0, 0, false, false, 0, false, 256>"
C5_TILE_N = 224               # output tile width the library takes for 4096 x 7168
# the kernels a default run times (the kernel-trace summary is of a default run); --all adds the
# split-K comparison's two
KERNEL_PATTERNS = (AQ_E4M3_KERNEL, AQ_E2M1_KERNEL, GEMM_FP8_FP4_KERNEL, GEMM_FP8_FP4_QUANT_KERNEL,
                   GEMM_FP8_FP8_KERNEL)
ALL_ONLY_PATTERNS = (GEMM_FP8_FP4_128_KERNEL, GEMM_FP8_FP4_SPLITK_KERNEL)
GEMM_THREADS = 256            # threads per workgroup of the 256x256-tile GEMM kernel
COPY_BYTES = 1 << 30          # the plain copy used to calibrate the HBM byte counters
COPY_REPS = 3                 # ... run this many times, last in the program


def _kernel_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, files):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of `kernel`, when it was
    taken on the current source (else None)."""
    p = os.path.join(HERE, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_hash") != _kernel_hash(files):
        return None
    return d.get("hbm_bytes_per_launch")


def _mfma_util(kernel: str, files):
    """MFMA utilisation of `kernel` (rocprofv3's MfmaUtil: MFMA-busy cycles over the SIMD cycles
    of the active GPU) from the committed counter summary, when it was taken on the current
    source (else None)."""
    p = os.path.join(HERE, "profiles", f"mfma_util_{kernel}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_hash") != _kernel_hash(files):
        return None
    return d.get("mfma_util")


def progress(msg: str):
    """One line per finished leg on stderr (the JSON result goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(fn, torch, ms: float | None = None) -> int:
    """Launches fn back to back for at least `ms` (default SETTLE_MS) of wall-clock time; returns
    the launch count."""
    ms = SETTLE_MS if ms is None else ms
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    batch = 1
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(batch):
            fn()
        n += batch
        torch.cuda.synchronize()
        batch = min(batch * 2, 256)
    return n


def median_ms(fn, torch, groups: int | None = None, per_group: int | None = None):
    """Median over `groups` groups of `per_group` back-to-back fn() calls of the time per call:
    one HIP event before the first group and one after each group, all on the current stream
    (the stream every launch here goes to), with no host synchronization in between, so each
    group's figure is the kernels' own time plus the short gaps between back-to-back dispatches
    and one event marker per group."""
    groups = GROUPS if groups is None else groups
    per_group = PER_GROUP if per_group is None else per_group
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    torch.cuda.synchronize()
    ev[0].record(s)
    for g in range(groups):
        for _ in range(per_group):
            fn()
        ev[g + 1].record(s)
    torch.cuda.synchronize()
    per = [ev[g].elapsed_time(ev[g + 1]) / per_group for g in range(groups)]
    return statistics.median(per), per


def timed(fn, torch):
    """settle() then median_ms(): (median ms per call, warm-up launches, timed launches)."""
    warm = settle(fn, torch)
    ms, _ = median_ms(fn, torch)
    return ms, warm, GROUPS * PER_GROUP


FLUSH_BYTES = 512 << 20        # written before each cold launch: twice the 256 MB last-level cache
COLD_ITERS = 10               # cold launches per leg (none in a counter run)


def cold_ms(fn, torch, flush, iters: int | None = None):
    """Median over `iters` (default COLD_ITERS) single calls of fn, each after the whole `flush`
    buffer (FLUSH_BYTES) was written, which evicts the L2s and the last-level cache: a pair of HIP
    events on the current stream around the call alone.  None when there are no iterations."""
    iters = COLD_ITERS if iters is None else iters
    if iters <= 0:
        return None
    cur = torch.cuda.current_stream()
    ts = []
    for i in range(iters):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        fn()
        b.record(cur)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return statistics.median(ts)


def paired_ms(fns, torch):
    """Median ms per call of each of `fns`, timed in alternation so that every one sees the same
    clock and temperature (the clock of this GPU moves with its recent load): a settling phase
    of at least SETTLE_MS that runs the functions in turn, then GROUPS rounds, each timing one
    group of PER_GROUP back-to-back calls of every function, in turn, with HIP events on the
    current stream."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for fn in fns:
            for _ in range(PER_GROUP):
                fn()
        torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    per = [[] for _ in fns]
    for _ in range(GROUPS):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        evs[0].record(st)
        for i, fn in enumerate(fns):
            for _ in range(PER_GROUP):
                fn()
            evs[i + 1].record(st)
        torch.cuda.synchronize()
        for i in range(len(fns)):
            per[i].append(evs[i].elapsed_time(evs[i + 1]) / PER_GROUP)
    return [statistics.median(x) for x in per]


def vendor_pair(torch, ours, batch, M, N, K):
    """The vendor library's plain bf16 GEMM (torch.matmul, which calls hipBLASLt) on the same
    shape, timed in alternation with our launch `ours` (paired_ms): what the bf16 MFMA reaches on
    this GPU with no decode and no scales, as context for the roofline fractions (not a path of
    this library)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    lead = () if batch is None else (batch,)
    a = torch.randn(lead + (M, K), device="cuda", dtype=torch.bfloat16, generator=g)
    # the right operand already [K, N] and contiguous: no transposed view reaches bmm
    b = torch.randn(lead + (K, N), device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(lead + (M, N), device="cuda", dtype=torch.bfloat16)

    def mm():
        torch.matmul(a, b, out=c)

    ours_ms, vendor_ms = paired_ms([ours, mm], torch)
    flops = 2.0 * M * N * K * (batch or 1)
    del a, b, c
    return {"vendor_ms": round(vendor_ms, 5),
            "vendor_tflops": round(flops / (vendor_ms * 1e-3) / 1e12, 2),
            "ours_ms": round(ours_ms, 5), "ours_over_vendor": round(vendor_ms / ours_ms, 4),
            "note": "torch.matmul (hipBLASLt) on bf16 N(0,1) operands of the same shape, timed "
                    "in alternation with this GEMM; ours_over_vendor = vendor time / our time"}


def gemm_roofline(ms, flops, peak_kind, kernel_desc, pattern, grid, warm, n, profile_key=None,
                  sources=GEMM_SOURCES):
    """Roofline block of one GEMM leg.  `grid` is the dispatch grid in work-items (x, y) as a
    kernel trace records it; `n` the number of timed launches, the last ones of that kernel and
    grid in the run."""
    tf = flops / (ms * 1e-3) / 1e12
    block = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS[peak_kind],
             "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS[peak_kind], 4),
             "traffic": _traffic(profile_key, sources) if profile_key else None,
             "kernel": kernel_desc, "median_launch_ms": round(ms, 5),
             "algorithmic_flops_per_launch": flops,
             "frac_of_bf16_peak": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4),
             "peak_note": f"peak is the dense {peak_kind.upper()} MFMA peak the operand formats name; "
                          "the kernel decodes them exactly to bf16 and runs the bf16 MFMA (2.5 PF), "
                          "because the FP8 MFMA adds mixed-exponent products inexactly and misses the "
                          "2^-20*sum|a*b| bound (tests/test_gpu_fp8_mfma_bound.py); frac_of_bf16_peak "
                          "is against the instruction it runs on",
             "timing": f"{warm} warm-up launches (>= {SETTLE_MS:.0f} ms), then the median of "
                       f"{GROUPS} groups of {PER_GROUP} back-to-back launches",
             "trace": {"kernel": pattern, "grid": list(grid), "last": n}}
    if profile_key:
        block["mfma_util"] = _mfma_util(profile_key, sources)
    return block


def cpu_baseline(w, rows: int, min_seconds: float = 10.0, max_runs: int = 30):
    """The oracle as it stands on the first `rows` rows of A (all of N and K), run again on the
    same sample until `min_seconds` of CPU work have accumulated (at least once, at most
    `max_runs` times); the rate is the mean over the runs."""
    from oracle import mx_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    runs, total, aq_total = 0, 0.0, 0.0
    while runs < max_runs and (runs == 0 or total < min_seconds):
        t0 = time.perf_counter()
        codes, sb = O.act_quant(w.x[:rows])
        aq_total += time.perf_counter() - t0
        A = O.decode_e4m3_rows(codes, sb)
        B = O.decode_fp4_rows(w.b, w.b_s)
        ref, S = O.gemm_ref(A, B, O.bf16_to_f64(w.bias))
        total += time.perf_counter() - t0
        runs += 1
        del codes, sb, A, B, ref, S
    dt = total / runs
    flops = 2.0 * rows * w.N * w.K
    aq_bytes = ACT_QUANT_BYTES_PER_ELEM * rows * w.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3), "runs": runs,
            "act_quant_gbs": round(aq_bytes / (aq_total / runs) / 1e9, 4),
            "act_quant_note": f"the oracle's act_quant alone on the same rows (numpy, one thread), "
                              f"{ACT_QUANT_BYTES_PER_ELEM} algorithmic bytes per element, mean "
                              f"over the same runs",
            "sample": f"act_quant + decode + float64 GEMM (with sum|a*b|) for rows 0..{rows - 1} of "
                      f"A [4096, 2048] against all 7168 weight rows, repeated {runs} times "
                      f"({total:.1f} s in all); flops counted as 2*{rows}*N*K per run"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--all", action="store_true", help="also the epilogue, split-K, backward and "
                    "A4W4 epilogue legs")
    ap.add_argument("--counter-run", action="store_true",
                    help="a short run for counter collection: 2 steps, no settling, one group of 2 "
                         "launches per leg, no CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-busy", metavar="BUSY_DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_busy:
        summarize_busy(args.summarize_busy)
        return
    if args.counter_run:
        global SETTLE_MS, GROUPS, PER_GROUP, COLD_ITERS
        SETTLE_MS, GROUPS, PER_GROUP, COLD_ITERS = 0.0, 1, 2, 0
        args.steps, args.warmup, args.no_cpu = 2, 1, True
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this hot path has no "
              f"multi-GPU leg", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_precision_act_amd as mx
    from block_scaled_precision_act_amd import synth

    mx.load()
    caps = mx.mx_capability()
    if not caps["available"]:
        print(f"no gfx950 device: {caps['reason']}", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def dev_u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    # ---- the step: act_quant -> FP8 x MXFP4 GEMM + bias on [4096, 2048] x [7168, 2048]
    w = synth.fp8xmxfp4_4096x7168x2048_bias()
    M, N, K = w.M, w.N, w.K
    x = dev_bf16(w.x)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    b, b_s, bias = dev_u8(w.b), dev_u8(w.b_s), dev_bf16(w.bias)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        mx.mx_act_quant(x, q, s, stream=stream)
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    progress(f"steps: {ms_per_step:.4f} ms per step")

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "e4m3xe2m1->bf16 mfma, f32 acc",
           "data": "synthetic (seeded numpy PCG64; no dataset)",
           "config": {"workload": "act_quant x[4096,2048] -> FP8xMXFP4 GEMM 4096x7168x2048 + bias",
                      "M": M, "N": N, "K": K, "x_outliers": "1% x100",
                      "weight_scales": "E8M0 118..136", "parallelism": "single GPU"}}

    # ---- variants of the step's GEMM on the same inputs (before the GEMM leg, so that the leg's
    # timed launches are the last of their kernel and grid in the run)
    out["next_layer_quant"] = bench_next_layer(mx, torch, q, s, b, b_s, bias, c, stream, flops)
    if args.all:
        out["epilogues"] = bench_epilogues(mx, torch, q, s, b, b_s, bias, c, stream, flops)

    # ---- the dominant kernel alone: the step's GEMM, settled, then the median per launch
    def gemm():
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias, stream=stream)

    # the cold launches and the vendor comparison first, so that the leg's own timed launches are
    # the last of the kernel
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    gemm_cold = cold_ms(gemm, torch, flush)
    del flush
    vendor = vendor_pair(torch, gemm, None, M, N, K)
    gemm_ms, warm, n = timed(gemm, torch)
    tiles = ((M + 255) // 256) * ((N + C5_TILE_N - 1) // C5_TILE_N)
    out["roofline"] = gemm_roofline(
        gemm_ms, flops, "fp8", "gemm_mx_kernel<fp8, fp4, bias> on 256x224 tiles (E4M3/E2M1 "
        "decoded exactly to bf16, bf16 MFMA)", GEMM_FP8_FP4_KERNEL, (tiles * GEMM_THREADS, 1), warm, n,
        "gemm_fp8_fp4_4096x7168x2048")
    out["gemm_only_tflops"] = out["roofline"]["achieved"]
    progress(f"gemm 4096x7168x2048: {gemm_ms * 1e3:.2f} us")
    out["roofline"]["vendor_bf16"] = vendor
    out["roofline"]["cold_ms"] = None if gemm_cold is None else round(gemm_cold, 5)
    del x

    # ---- the two large FP8 x FP8 configurations (A quantized on the GPU by act_quant)
    out["gemm_8192cubed"] = bench_large(mx, synth, torch, dev_u8, dev_bf16, stream,
                                        synth.fp8xfp8_8192cubed(), "gemm_fp8_fp8_8192cubed")
    out["gemm_batched_8x1024x2048x2048"] = bench_large(
        mx, synth, torch, dev_u8, dev_bf16, stream, synth.fp8xfp8_batched_8x1024x2048x2048(),
        "gemm_fp8_fp8_batched_8x1024x2048x2048")
    progress("large fp8 x fp8 gemms done")


    # ---- the latency-bound configurations
    out["latency"] = bench_latency(mx, synth, torch, dev_u8, dev_bf16, stream, args.all)
    progress("small configurations done")

    # ---- standalone producers on [16384, 7168]
    out["act_quant"], out["act_quant_fp4"] = bench_act_quant(mx, synth, torch, dev_bf16, stream)
    progress("producers done")

    if args.all:
        out["splitk"] = bench_splitk(mx, synth, torch, dev_u8, dev_bf16, stream)
        out["backward"] = bench_backward(mx, synth, torch, dev_bf16, w.x, stream)

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


def bench_next_layer(mx, torch, q, s, b, b_s, bias, c, stream, flops):
    """The step's GEMM emitting the next layer's activation operand (E4M3 codes + per-32 E8M0
    bytes of the bf16 output) against the bf16 GEMM followed by act_quant on its output."""
    M, N = c.shape
    qn = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    qsn = torch.empty((M, N // 32), dtype=torch.uint8, device="cuda")

    def fused():
        mx.mx_gemm_fp8_fp4_quant(q, s, b, b_s, qn, qsn, bias=bias, stream=stream)

    def unfused():
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias, stream=stream)
        mx.mx_act_quant(c, qn, qsn, stream=stream)

    fused_ms, unfused_ms = paired_ms([fused, unfused], torch)
    return {"workload": "FP8xMXFP4 GEMM 4096x7168x2048 + bias -> E4M3 [4096, 7168] + "
                        "E8M0 [4096, 224] for the next layer",
            "fused_ms": round(fused_ms, 5), "unfused_ms": round(unfused_ms, 5),
            "fused_tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
            "speedup": round(unfused_ms / fused_ms, 3),
            "fused_traffic": _traffic("gemm_fp8_fp4_quant_4096x7168x2048", GEMM_SOURCES)}


def bench_epilogues(mx, torch, q, s, b, b_s, bias, c, stream, flops):
    """The residual and GELU epilogues on the step's GEMM (bf16 out)."""
    res_t = torch.empty(c.shape, dtype=torch.bfloat16, device="cuda").normal_()

    def with_residual():
        mx.mx_gemm_fp8_fp4_bias_residual(q, s, b, b_s, res_t, c, bias=bias, stream=stream)

    def with_gelu():
        mx.mx_gemm_fp8_fp4_bias_gelu(q, s, b, b_s, c, bias=bias, stream=stream)

    res_ms, _, _ = timed(with_residual, torch)
    gelu_ms, _, _ = timed(with_gelu, torch)
    return {"workload": "FP8xMXFP4 GEMM 4096x7168x2048 + bias, bf16 out: + bf16 residual "
                        "[4096, 7168], or GELU",
            "bias_residual_ms": round(res_ms, 5),
            "bias_residual_tflops": round(flops / (res_ms * 1e-3) / 1e12, 2),
            "bias_gelu_ms": round(gelu_ms, 5),
            "bias_gelu_tflops": round(flops / (gelu_ms * 1e-3) / 1e12, 2)}


def bench_large(mx, synth, torch, dev_u8, dev_bf16, stream, w, profile_key):
    """One large FP8 x FP8 (32x32 block-scaled weight) configuration: act_quant of its
    activations on the GPU, then the GEMM leg with its own roofline block."""
    xq = dev_bf16(w.x)
    a = torch.empty(xq.shape, dtype=torch.uint8, device="cuda")
    a_s = torch.empty(xq.shape[:-1] + (xq.shape[-1] // 32,), dtype=torch.uint8, device="cuda")
    if xq.dim() == 3:
        mx.mx_act_quant_strided_batched(xq, a, a_s, stream=stream)
    else:
        mx.mx_act_quant(xq, a, a_s, stream=stream)
    del xq
    b, b_s = dev_u8(w.b), dev_u8(w.b_s)
    batch = w.batch or 1
    shape = (w.M, w.N) if w.batch is None else (w.batch, w.M, w.N)
    c = torch.empty(shape, dtype=torch.bfloat16, device="cuda")

    def gemm():
        mx.mx_gemm_fp8_fp8(a, a_s, b, b_s, c, stream=stream)

    # the cold launches and the vendor comparison first, so that the leg's own timed launches are
    # the last of the kernel and grid
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    cold = cold_ms(gemm, torch, flush)
    del flush
    vendor = vendor_pair(torch, gemm, w.batch, w.M, w.N, w.K)
    ms, warm, n = timed(gemm, torch)
    flops = 2.0 * w.M * w.N * w.K * batch
    tiles = ((w.M + 255) // 256) * ((w.N + 255) // 256)
    block = gemm_roofline(ms, flops, "fp8", "gemm_mx_kernel<fp8, fp8> (E4M3 decoded exactly to "
                          "bf16, bf16 MFMA)", GEMM_FP8_FP8_KERNEL, (tiles * GEMM_THREADS, batch),
                          warm, n, profile_key)
    batch_txt = f"{w.batch} x " if w.batch else ""
    block["workload"] = (f"FP8xFP8 GEMM {batch_txt}{w.M}x{w.N}x{w.K}, 32x32 block-scaled E4M3 "
                         f"weights, activations through act_quant, no bias")
    block["vendor_bf16"] = vendor
    block["cold_ms"] = None if cold is None else round(cold, 5)
    del a, a_s, b, b_s, c
    return block


def bench_latency(mx, synth, torch, dev_u8, dev_bf16, stream, epilogues=False):
    """The small configurations, for which launch latency and caches matter: the median per
    launch (as every other leg), `graph_ms` (20 launches captured in one HIP graph and replayed
    10 times: launch overhead amortized) and `cold_ms` (median of 10 single launches, each after
    512 MB were written to evict the caches; events around the GEMM alone)."""
    res = {}
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def graph_ms(launch, reps=20, iters=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                launch(None)                  # the capture stream is the current stream
        g.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(cur)
        for _ in range(iters):
            g.replay()
        end.record(cur)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / (iters * reps)

    def run(w, kind, hbm=False):
        if w.a_kind == "acts":
            xq = dev_bf16(w.x)
            a = torch.empty(xq.shape, dtype=torch.uint8, device="cuda")
            a_s = torch.empty(xq.shape[:-1] + (xq.shape[-1] // 32,), dtype=torch.uint8, device="cuda")
            mx.mx_act_quant(xq, a, a_s, stream=stream)
            del xq
        else:
            a, a_s = dev_u8(w.a), dev_u8(w.a_s)
        b, b_s = dev_u8(w.b), dev_u8(w.b_s)
        bias_t = dev_bf16(w.bias) if w.bias is not None else None
        c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        fn = getattr(mx, f"mx_gemm_{kind}")

        def launch(st):
            fn(a, a_s, b, b_s, c, bias=bias_t, stream=st)

        ms, _, _ = timed(lambda: launch(stream), torch)
        flops = 2.0 * w.M * w.N * w.K
        r = {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
             "graph_ms": round(graph_ms(launch), 5),
             "cold_ms": cold_ms(lambda: launch(stream), torch, flush)}
        if r["cold_ms"] is not None:
            r["cold_ms"] = round(r["cold_ms"], 5)
        r["graph_tflops"] = round(flops / (r["graph_ms"] * 1e-3) / 1e12, 3)
        if hbm:
            nbytes = (w.M * w.K / 2 + w.M * w.K / 32 + w.N * w.K / 2 + w.N * w.K / 32 +
                      2 * w.M * w.N)
            r["algorithmic_bytes"] = nbytes
            r["gbs"] = round(nbytes / (r["ms"] * 1e-3) / 1e9, 1)
            r["graph_gbs"] = round(nbytes / (r["graph_ms"] * 1e-3) / 1e9, 1)
            r["cold_gbs"] = (None if r["cold_ms"] is None else
                             round(nbytes / (r["cold_ms"] * 1e-3) / 1e9, 1))
            r["graph_frac_of_hbm"] = round(r["graph_gbs"] / HBM_PEAK_GBS, 4)
        if epilogues and kind == "fp4_fp4":
            r.update(bench_a4w4_epilogues(mx, torch, a, a_s, b, b_s, bias_t, c, w, kind, stream))
        return r

    res["fp8xmxfp4_16x256x512"] = run(synth.fp8xmxfp4_16x256x512(), "fp8_fp4")
    res["fp8xfp8_1024^3_bias"] = run(synth.fp8xfp8_1024cubed_bias(), "fp8_fp8")
    for i in range(3):
        w = synth.a4w4_skinny(i)
        res[w.name] = run(w, "fp4_fp4", hbm=True)
    del flush
    return res


def bench_a4w4_epilogues(mx, torch, a, a_s, b, b_s, bias_t, c, w, kind, stream):
    """Residual and GELU epilogues of one A4W4 shape, and bias + GELU written as packed MXFP4 for
    the next A4W4 layer, fused and as GELU then the MXFP4 producer."""
    r = {}
    resid = torch.empty(c.shape, dtype=torch.bfloat16, device="cuda").normal_()
    fr = getattr(mx, f"mx_gemm_{kind}_bias_residual")
    fg = getattr(mx, f"mx_gemm_{kind}_bias_gelu")
    r["bias_residual_ms"] = round(timed(
        lambda: fr(a, a_s, b, b_s, resid, c, bias=bias_t, stream=stream), torch)[0], 5)
    r["bias_gelu_ms"] = round(timed(
        lambda: fg(a, a_s, b, b_s, c, bias=bias_t, stream=stream), torch)[0], 5)
    qn = torch.empty((w.M, w.N // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((w.M, w.N // 32), dtype=torch.uint8, device="cuda")
    fq = getattr(mx, f"mx_gemm_{kind}_bias_gelu_quant")

    def unfused():
        fg(a, a_s, b, b_s, c, bias=bias_t, stream=stream)
        mx.mx_act_quant_fp4(c, qn, qs, stream=stream)

    r["bias_gelu_quant_ms"] = round(timed(
        lambda: fq(a, a_s, b, b_s, qn, qs, bias=bias_t, stream=stream), torch)[0], 5)
    r["bias_gelu_then_quant_ms"] = round(timed(unfused, torch)[0], 5)
    return r


def bench_act_quant(mx, synth, torch, dev_bf16, stream):
    """Standalone act_quant and MXFP4 producer on [16384, 7168], sustained: back-to-back
    launches rotating over three input/output sets (1.07 GB, far beyond the 256 MB last-level
    cache), so each launch reads its input from HBM and pays for the previous launch's
    write-back."""
    xs_bits = synth.act_quant_standalone_16384x7168()
    xs = [dev_bf16(xs_bits)]
    del xs_bits
    xs += [xs[0].clone() for _ in range(2)]
    rows, cols = xs[0].shape
    qs = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda") for _ in range(3)]
    ss = [torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda") for _ in range(3)]
    rot = [0]

    def aq_launch():
        i = rot[0] % 3
        rot[0] += 1
        mx.mx_act_quant(xs[i], qs[i], ss[i], stream=stream)

    aq_ms, warm, n = timed(aq_launch, torch)
    aq_bytes = ACT_QUANT_BYTES_PER_ELEM * rows * cols
    aq_gbs = aq_bytes / (aq_ms * 1e-3) / 1e9
    aq = {"workload": "act_quant bf16 [16384, 7168] -> E4M3 + E8M0 (3 rotating buffer sets)",
          "value": round(aq_gbs, 1), "unit": "GB/s", "median_launch_ms": round(aq_ms, 5),
          "roofline": {"bound": "hbm", "achieved": round(aq_gbs, 1), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(aq_gbs / HBM_PEAK_GBS, 4),
                       "traffic": _traffic("act_quant_16384x7168", ACT_QUANT_SOURCES),
                       "algorithmic_bytes_per_launch": aq_bytes,
                       "timing": f"{warm} warm-up launches (>= {SETTLE_MS:.0f} ms), then the median "
                                 f"of {GROUPS} groups of {PER_GROUP} back-to-back launches",
                       "trace": {"kernel": AQ_E4M3_KERNEL, "grid": None, "last": n}}}
    del qs
    q4 = [torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda") for _ in range(3)]

    def aq4_launch():
        i = rot[0] % 3
        rot[0] += 1
        mx.mx_act_quant_fp4(xs[i], q4[i], ss[i], stream=stream)

    aq4_ms, warm, n = timed(aq4_launch, torch)
    aq4_bytes = ACT_QUANT_FP4_BYTES_PER_ELEM * rows * cols
    aq4_gbs = aq4_bytes / (aq4_ms * 1e-3) / 1e9
    aq4 = {"workload": "act_quant_fp4 bf16 [16384, 7168] -> packed E2M1 + E8M0 "
                       "(3 rotating buffer sets)",
           "value": round(aq4_gbs, 1), "unit": "GB/s", "median_launch_ms": round(aq4_ms, 5),
           "roofline": {"bound": "hbm", "achieved": round(aq4_gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(aq4_gbs / HBM_PEAK_GBS, 4),
                        "traffic": _traffic("act_quant_fp4_16384x7168", ACT_QUANT_SOURCES),
                        "algorithmic_bytes_per_launch": aq4_bytes,
                        "timing": f"{warm} warm-up launches (>= {SETTLE_MS:.0f} ms), then the "
                                  f"median of {GROUPS} groups of {PER_GROUP} back-to-back launches",
                        "trace": {"kernel": AQ_E2M1_KERNEL, "grid": None, "last": n}}}
    del xs, q4, ss
    return aq, aq4


def bench_splitk(mx, synth, torch, dev_u8, dev_bf16, stream):
    """Split-K on the down-projection shape 4096x2048x7168 (128 output tiles of 256x256 for 256
    CUs): the same inputs through the plain and the split-K entry point."""
    wd = synth.gemm_inputs("fp8", "fp4", 4096, 2048, 7168, 1006, with_bias=True,
                           name="fp8xmxfp4_m4096_n2048_k7168_bias")
    ad, asd, bd, bsd = dev_u8(wd.a), dev_u8(wd.a_s), dev_u8(wd.b), dev_u8(wd.b_s)
    biasd = dev_bf16(wd.bias)
    cd = torch.empty((wd.M, wd.N), dtype=torch.bfloat16, device="cuda")
    wsd = torch.zeros(mx.mx_gemm_splitk_workspace_size(wd.M, wd.N, wd.K), dtype=torch.uint8,
                      device="cuda")

    def down_plain():
        mx.mx_gemm_fp8_fp4(ad, asd, bd, bsd, cd, bias=biasd, stream=stream)

    def down_split():
        mx.mx_gemm_fp8_fp4_splitk(ad, asd, bd, bsd, cd, wsd, bias=biasd, stream=stream)

    dflops = 2.0 * wd.M * wd.N * wd.K
    plain_ms = timed(down_plain, torch)[0]
    split_ms = timed(down_split, torch)[0]
    return {"workload": "FP8xMXFP4 GEMM 4096x2048x7168 + bias (128 tiles of 256x256): plain "
                        "launch against K split in two",
            "plain_ms": round(plain_ms, 5), "plain_tflops": round(dflops / (plain_ms * 1e-3) / 1e12, 2),
            "splitk_ms": round(split_ms, 5), "splitk_tflops": round(dflops / (split_ms * 1e-3) / 1e12, 2),
            "speedup": round(plain_ms / split_ms, 3), "workspace_bytes": int(wsd.numel())}


def bench_backward(mx, synth, torch, dev_bf16, x_bits, stream):
    """dX and dW of the 4096x7168x2048 linear layer: each kernel, then the whole six-kernel
    backward step, timed as every leg is (settled, then the median per launch)."""
    M, K = x_bits.shape
    N = 7168
    rng = synth.rng_for(1007)
    W = dev_bf16(synth.bf16_normal(rng, (N, K), std=0.05))
    dY = dev_bf16(synth.bf16_normal(rng, (M, N), std=1e-3))
    x = dev_bf16(x_bits)
    u8 = dict(dtype=torch.uint8, device="cuda")
    gq, gs = torch.empty((M, N), **u8), torch.empty((M, N // 32), **u8)
    wq, wsc = torch.empty((K, N), **u8), torch.empty((K, N // 32), **u8)
    gtq, gts = torch.empty((N, M), **u8), torch.empty((N, M // 32), **u8)
    xq, xs = torch.empty((K, M), **u8), torch.empty((K, M // 32), **u8)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(mx.mx_gemm_splitk_workspace_size(M, K, N), 256), **u8)
    steps = {
        "quant_e5m2_dY": lambda: mx.mx_quant_e5m2(dY, gq, gs, seed=1234, stream=stream),
        "quant_transpose_e4m3_W": lambda: mx.mx_quant_transpose_e4m3(W, wq, wsc, stream=stream),
        "gemm_dX_splitk": lambda: mx.mx_gemm_e5m2_e4m3_splitk(gq, gs, wq, wsc, dX, ws, stream=stream),
        "quant_transpose_e5m2_dY": lambda: mx.mx_quant_transpose_e5m2(dY, gtq, gts, seed=4321,
                                                                      stream=stream),
        "quant_transpose_e4m3_x": lambda: mx.mx_quant_transpose_e4m3(x, xq, xs, stream=stream),
        "gemm_dW": lambda: mx.mx_gemm_e5m2_e4m3(gtq, gts, xq, xs, dW, stream=stream),
    }

    def step():
        for f in steps.values():
            f()

    res = {"workload": "backward of y = x W^T, x [4096, 2048], W [7168, 2048], dY [4096, 7168]: "
                       "dX = dY W (K split), dW = dY^T x; stochastic E5M2 gradients"}
    qbytes = {"quant_e5m2_dY": M * N, "quant_transpose_e4m3_W": N * K,
              "quant_transpose_e5m2_dY": M * N, "quant_transpose_e4m3_x": M * K}
    flops = 2.0 * M * N * K
    for name, f in steps.items():
        ms = timed(f, torch)[0]
        entry = {"ms": round(ms, 5)}
        if name in qbytes:
            entry["gbs"] = round(ACT_QUANT_BYTES_PER_ELEM * qbytes[name] / (ms * 1e-3) / 1e9, 1)
        else:
            entry["tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
        res[name] = entry
    rne_ms = timed(lambda: mx.mx_quant_e5m2(dY, gq, gs, stream=stream), torch)[0]
    res["quant_e5m2_dY_round_to_nearest"] = {
        "ms": round(rne_ms, 5), "gbs": round(ACT_QUANT_BYTES_PER_ELEM * M * N / (rne_ms * 1e-3) / 1e9, 1)}
    step_ms = timed(step, torch)[0]
    res["step_ms"] = round(step_ms, 5)
    res["step_tflops"] = round(2 * flops / (step_ms * 1e-3) / 1e12, 2)
    return res


def _bench_line(stats_dir):
    """The JSON line bench.py printed in the traced run (saved as bench_stdout.txt)."""
    p = os.path.join(stats_dir, "bench_stdout.txt")
    if not os.path.exists(p):
        return {}
    with open(p) as fh:
        js = [ln for ln in fh if ln.startswith("{")]
    return json.loads(js[-1]) if js else {}


def _roofline_blocks(line):
    """(name, block) of every block of the line that carries a `trace` selector."""
    out = []
    if "roofline" in line:
        out.append(("gemm_fp8_fp4 4096x7168x2048 + bias", line["roofline"]))
    for key in ("gemm_8192cubed", "gemm_batched_8x1024x2048x2048"):
        if key in line:
            out.append((key, line[key]))
    for key in ("act_quant", "act_quant_fp4"):
        if key in line and "roofline" in line[key]:
            blk = dict(line[key]["roofline"])
            blk["median_launch_ms"] = line[key].get("median_launch_ms")
            out.append((key + " [16384, 7168]", blk))
    return out


def trace_check(stats_dir):
    """For every roofline block of the traced run's line: the kernel-trace durations of the
    dispatches it timed (the last `last` dispatches of its kernel and grid), against the median
    per launch the line reports from HIP events."""
    import csv
    import glob
    line = _bench_line(stats_dir)
    seq = []
    for f in glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                seq.append((int(r["Start_Timestamp"]), r["Kernel_Name"],
                            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                            int(r["Grid_Size_X"]), int(r["Grid_Size_Y"])))
    seq.sort()
    res = {}
    for name, blk in _roofline_blocks(line):
        tr = blk.get("trace") or {}
        pat, grid, last = tr.get("kernel"), tr.get("grid"), tr.get("last")
        if not pat or not last:
            continue
        d = [dur / 1000.0 for _, k, dur, gx, gy in seq
             if re.search(pat, k) and (grid is None or (gx, gy) == tuple(grid))]
        d = d[-last:]
        if len(d) < last:
            continue
        ev = blk.get("median_launch_ms")
        res[name] = {"dispatches": len(d), "trace_mean_us": sum(d) / len(d),
                     "trace_median_us": statistics.median(d),
                     "events_median_us": None if ev is None else ev * 1e3}
    return res


def summarize(stats_dir, fetch_dir, write_dir):
    """Writes the profiles/ summaries from rocprofv3 CSV output of this script: kernel-trace
    stats of a default run (with its timed dispatches matched against the line it printed), and
    FETCH_SIZE / WRITE_SIZE per dispatch scaled by what the same counters read for the plain
    1 GiB copy (--copy-calibration)."""
    import csv
    import glob

    def rows(d, pattern):
        out = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    stats = rows(stats_dir, "*kernel_stats.csv")
    prof = os.path.join(HERE, "profiles")
    os.makedirs(prof, exist_ok=True)

    def per_dispatch(d, counter):
        vals = {}
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Grid_Size"]), r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0   # KiB -> bytes
        return vals

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")

    def pick(vals, name_part, grid=None):
        v = [b for (k, g, _), b in vals.items()
             if re.search(name_part, k) and (grid is None or g == grid)]
        return sum(v) / len(v) if v else None

    def calib(vals):
        # the calibration copies are the last COPY_REPS copyBuffer dispatches of the run (the
        # input uploads before them can have the same grid but move fewer bytes)
        cands = sorted((int(d), b) for (k, _, d), b in vals.items() if "copyBuffer" in k)
        if len(cands) < COPY_REPS:
            return None
        v = [b for _, b in cands[-COPY_REPS:]]
        return sum(v) / len(v)

    copy_f, copy_w = calib(fetch), calib(write)
    f_factor = copy_f / COPY_BYTES if copy_f else None
    w_factor = copy_w / COPY_BYTES if copy_w else None
    # act_quant on [16384, 7168]: the E4M3 act_quant dispatches with the largest grid
    aq8, aq4 = AQ_E4M3_KERNEL, AQ_E2M1_KERNEL
    aq_grids = [g for (k, g, _) in list(fetch) + list(write) if re.search(aq8, k)]
    aq_grid = max(aq_grids) if aq_grids else None
    aq4_grids = [g for (k, g, _) in list(fetch) + list(write) if re.search(aq4, k)]
    aq4_grid = max(aq4_grids) if aq4_grids else None
    aq_alg = ACT_QUANT_BYTES_PER_ELEM * 16384 * 7168
    aq4_alg = ACT_QUANT_FP4_BYTES_PER_ELEM * 16384 * 7168
    gemm_in = 4096 * 2048 + 4096 * 64 + 7168 * 1024 + 7168 * 64 + 2 * 7168
    gemm_alg = gemm_in + 2 * 4096 * 7168
    gemm_q_alg = gemm_in + 4096 * 7168 + 4096 * 7168 // 32

    def fp8_alg(batch, m, n, k):       # E4M3 A + scales, E4M3 B + 32x32 scales, bf16 C
        return batch * (m * k + m * k // 32 + n * k + (n // 32) * (k // 32) + 2 * m * n)

    # the split-K line's down-projection 4096x2048x7168 (its partial tiles are not algorithmic)
    down_alg = 4096 * 7168 + 4096 * 224 + 2048 * 3584 + 2048 * 224 + 2 * 2048 + 2 * 4096 * 2048
    grid8192 = 32 * 32 * GEMM_THREADS
    grid_b8 = 4 * 8 * GEMM_THREADS * 8
    out = {}
    for name, part, grid, files, alg in (
            ("act_quant_16384x7168", aq8, aq_grid, ACT_QUANT_SOURCES, aq_alg),
            ("act_quant_fp4_16384x7168", aq4, aq4_grid, ACT_QUANT_SOURCES, aq4_alg),
            ("gemm_fp8_fp4_4096x7168x2048", GEMM_FP8_FP4_KERNEL, None,
             GEMM_SOURCES, gemm_alg),
            ("gemm_fp8_fp4_quant_4096x7168x2048", GEMM_FP8_FP4_QUANT_KERNEL, None,
             GEMM_SOURCES, gemm_q_alg),
            ("gemm_fp8_fp8_8192cubed", GEMM_FP8_FP8_KERNEL, grid8192, GEMM_SOURCES,
             fp8_alg(1, 8192, 8192, 8192)),
            ("gemm_fp8_fp8_batched_8x1024x2048x2048", GEMM_FP8_FP8_KERNEL, grid_b8,
             GEMM_SOURCES, fp8_alg(8, 1024, 2048, 2048)),
            ("gemm_fp8_fp4_4096x2048x7168_plain", GEMM_FP8_FP4_128_KERNEL,
             None, GEMM_SOURCES, down_alg),
            ("gemm_fp8_fp4_4096x2048x7168_splitk", GEMM_FP8_FP4_SPLITK_KERNEL,
             None, GEMM_SOURCES, down_alg)):
        f, w = pick(fetch, part, grid), pick(write, part, grid)
        if f is None or w is None or not f_factor or not w_factor:
            continue
        hbm = f / f_factor + w / w_factor
        out[name] = {"source_hash": _kernel_hash(files), "fetch_bytes_raw": f, "write_bytes_raw": w,
                     "fetch_scale": f_factor, "write_scale": w_factor,
                     "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": alg,
                     "traffic_over_algorithmic": round(hbm / alg, 3)}
        with open(os.path.join(prof, f"traffic_{name}.json"), "w") as fh:
            json.dump(out[name], fh, indent=1)
    checks = trace_check(stats_dir)
    cmds = {
        "stats": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/stats -o run "
                 "-- python3 bench.py > OUT/stats/bench_stdout.txt",
        "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run "
                 "-- python3 bench.py --counter-run --copy-calibration --all",
        "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run "
                 "-- python3 bench.py --counter-run --copy-calibration --all",
        "summary": "python bench.py --summarize OUT/stats OUT/fetch OUT/write",
    }
    lines = ["rocprofv3 kernel-trace statistics of one bench.py run at its default settings",
             "(the act_quant -> FP8xMXFP4 GEMM 4096x7168x2048 + bias steps, then every timed leg of",
             "the line: the next-layer quantized GEMM, the GEMM alone, the 8192^3 and batched",
             "8x1024x2048x2048 FP8xFP8 GEMMs, the small configurations, and the standalone producers",
             "on [16384, 7168]; each leg settles for >= 100 ms, then times 12 groups of 10 launches).",
             "", "command: " + cmds["stats"],
             "(TMPDIR=/tmp, repository root as cwd, OUT the folder the profiler writes to)", ""]
    if stats:
        keys = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "StdDev", "Percentage"]
        lines.append(" | ".join(keys))
        for r in stats:
            name = r.get("Name", "")
            if len(name) > 160:
                name = name[:157] + "..."
            lines.append(" | ".join([name] + [str(r.get(k, "")) for k in keys[1:]]))
    if checks:
        lines += ["", "Timed dispatches of each roofline block (the last dispatches of its kernel and",
                  "grid, as many as it timed), from the kernel trace of the same run, beside the",
                  "median per launch the run's bench.py line reports from HIP events:"]
        for name, d in checks.items():
            ev = "n/a" if d["events_median_us"] is None else f"{d['events_median_us']:.2f} us"
            lines.append(f"  {name}: {d['dispatches']} dispatches, trace mean "
                         f"{d['trace_mean_us']:.2f} us, trace median {d['trace_median_us']:.2f} us, "
                         f"events median {ev}")
    with open(os.path.join(prof, "kernel_stats_bench_default_run.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    tl = ["HBM traffic per launch from rocprofv3 --pmc (FETCH_SIZE and WRITE_SIZE in separate runs),",
          "each scaled by what the same counter reads for a plain 1 GiB device copy",
          f"(FETCH_SIZE/bytes = {f_factor}, WRITE_SIZE/bytes = {w_factor}).", "",
          "commands (OUT: the folder the profiler writes to):", "  " + cmds["fetch"],
          "  " + cmds["write"], "  " + cmds["summary"], ""]
    for name, d in out.items():
        tl.append(f"{name}: hbm_bytes_per_launch = {d['hbm_bytes_per_launch']}, algorithmic = "
                  f"{d['algorithmic_bytes_per_launch']:.0f}, ratio = {d['traffic_over_algorithmic']} "
                  f"(fetch {d['fetch_bytes_raw'] / d['fetch_scale']:.0f} B, write "
                  f"{d['write_bytes_raw'] / d['write_scale']:.0f} B; source hash {d['source_hash']})")
    if out:
        with open(os.path.join(prof, "traffic_bench_kernels.txt"), "w") as fh:
            fh.write("\n".join(tl) + "\n")
    print("\n".join(lines + [""] + tl))


BUSY_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE "
                 "SQ_INSTS_MFMA")


# the GEMMs whose MFMA utilisation the counter run records: profile key, title, kernel pattern,
# dispatch grid in work-items (None: the only grid of that kernel in the run), batch, M, N, K
BUSY_TARGETS = (
    ("gemm_fp8_fp4_4096x7168x2048", "the FP8xMXFP4 GEMM 4096x7168x2048 + bias",
     GEMM_FP8_FP4_KERNEL, None, 1, 4096, 7168, 2048),
    ("gemm_fp8_fp8_8192cubed", "the FP8xFP8 GEMM 8192^3",
     GEMM_FP8_FP8_KERNEL, 32 * 32 * GEMM_THREADS, 1, 8192, 8192, 8192),
    ("gemm_fp8_fp8_batched_8x1024x2048x2048", "the FP8xFP8 GEMM 8 x 1024x2048x2048",
     GEMM_FP8_FP8_KERNEL, 4 * 8 * GEMM_THREADS * 8, 8, 1024, 2048, 2048),
)


def summarize_busy(busy_dir, prof_dir=None):
    """MFMA utilisation of the large GEMMs (BUSY_TARGETS) from one rocprofv3 --pmc run of
    BUSY_COUNTERS with --kernel-trace (the trace gives each dispatch's duration).  Counter values
    in the csv are sums over the XCDs and shader engines.  Per dispatch:
    * active cycles g = GRBM_GUI_ACTIVE / XCDs (the GUI counter runs once per XCD), clock = g / ns;
    * mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (g * SIMDs), rocprofv3's own MfmaUtil;
    * cu_busy = SQ_BUSY_CU_CYCLES / (g * CUs), and mfma_busy_over_busy_cu = MFMA-busy cycles over
      the SIMD cycles of CUs that hold a workgroup.  SQ_BUSY_CU_CYCLES is read in plain cycles:
      read as quad-cycles it would exceed CUs * g threefold.
    Medians over each GEMM's dispatches are written to mfma_util_<key>.json and .txt in prof_dir
    (profiles/ by default); the 4096x7168x2048 GEMM's figures are returned."""
    import csv
    import glob
    import statistics

    def rows(pattern):
        files = glob.glob(os.path.join(busy_dir, "**", pattern), recursive=True)
        return [r for f in files for r in csv.DictReader(open(f))]

    agent = [r for r in rows("*agent_info.csv") if r.get("Name", "").startswith("gfx")][0]
    simds, cus, xcds = int(agent["Simd_Count"]), int(agent["Cu_Count"]), int(agent["Num_Xcc"])
    dur = {r["Dispatch_Id"]: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
           for r in rows("*kernel_trace.csv")}
    counter_rows = rows("*counter_collection.csv")
    cmd = (f"rocprofv3 --pmc {BUSY_COUNTERS} --kernel-trace --output-format csv -d OUT/busy -o run "
           "-- python3 bench.py --counter-run")
    prof = prof_dir or os.path.join(HERE, "profiles")
    result = None
    for key, title, pattern, grid, batch, M, N, K in BUSY_TARGETS:
        ctr = {}
        for r in counter_rows:
            if not re.search(pattern, r["Kernel_Name"]):
                continue
            if grid is not None and int(r.get("Grid_Size", -1)) != grid:
                continue
            ctr.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
        per = []
        for did, v in ctr.items():
            if did not in dur or len(v) < len(BUSY_COUNTERS.split()):
                continue
            g = v["GRBM_GUI_ACTIVE"] / xcds
            per.append({"duration_us": dur[did] / 1000.0, "clock_ghz": g / dur[did],
                        "mfma_util": v["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * simds),
                        "cu_busy": v["SQ_BUSY_CU_CYCLES"] / (g * cus),
                        "mfma_busy_over_busy_cu": v["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                  (v["SQ_BUSY_CU_CYCLES"] * simds / cus),
                        "mfma_insts": v["SQ_INSTS_MFMA"],
                        "mfma_busy_cycles_per_inst": v["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                                     v["SQ_INSTS_MFMA"]})
        if not per:
            print(f"{key}: no dispatches with every counter found", file=sys.stderr)
            continue
        med = {k: round(statistics.median(d[k] for d in per), 4) for k in per[0]}
        out = {"source_hash": _kernel_hash(GEMM_SOURCES), "dispatches": len(per),
               "simds": simds, "cus": cus, "xcds": xcds,
               "mfma_insts_expected": 2 * batch * M * N * K // (32 * 32 * 16 * 2), **med,
               "command": cmd}
        with open(os.path.join(prof, f"mfma_util_{key}.json"), "w") as fh:
            json.dump(out, fh, indent=1)
        txt = [f"MFMA utilisation of {title} (bf16 MFMA 32x32x16),",
               f"medians over {len(per)} dispatches of one counter run:", "",
               "command (TMPDIR=/tmp, repository root as cwd, OUT the folder the profiler writes to):",
               "  " + cmd, "  python bench.py --summarize-busy OUT/busy", "",
               f"duration {med['duration_us']} us at {med['clock_ghz']} GHz "
               f"(GRBM_GUI_ACTIVE over the {xcds} XCDs / duration)",
               f"MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x {simds} SIMDs) = "
               f"{med['mfma_util']}",
               f"CUs holding a workgroup: {med['cu_busy']} of the active cycles; MFMA-busy over their "
               f"SIMD cycles = {med['mfma_busy_over_busy_cu']}",
               f"MFMA instructions {med['mfma_insts']:.0f} (2MNK/32768 = "
               f"{out['mfma_insts_expected']}), {med['mfma_busy_cycles_per_inst']} busy cycles each",
               f"source hash {out['source_hash']}"]
        with open(os.path.join(prof, f"mfma_util_{key}.txt"), "w") as fh:
            fh.write("\n".join(txt) + "\n")
        print("\n".join(txt) + "\n")
        if result is None and key == BUSY_TARGETS[0][0]:
            result = out
    return result


if __name__ == "__main__":
    main()
