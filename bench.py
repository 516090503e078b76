"""Benchmark of the microscaled hot path on one MI355X.

One step is the whole path on one batch of synthetic input, back to back on one stream:
act_quant of bf16 activations x [4096, 2048] (N(0,1) with 1% of entries x100) into E4M3 codes +
E8M0 scales, then the FP8 x MXFP4 GEMM against E2M1 weights [7168, 2048] (per-32 E8M0 scales
118..136) with a fused bf16 bias, bf16 out [4096, 7168].

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all]
    python bench.py --summarize STATS_DIR FETCH_DIR WRITE_DIR   (CPU only; writes profiles/)
    python bench.py --summarize-busy BUSY_DIR                   (CPU only; writes profiles/)

Prints one JSON line.  `value` is the GEMM's 2*M*N*K flops divided by the time of a whole step
(act_quant included), in TFLOP/s.  `roofline` is the dominant kernel (the GEMM): as many
back-to-back launches of it as there are steps, on the step's stream and inputs, bracketed by one
pair of HIP events on that stream.  `act_quant` reports the standalone producer on [16384, 7168]
against HBM bandwidth, `act_quant_fp4` the MXFP4 producer on the same input.  `cpu_baseline`
times the oracle on a bounded sample of the same workload on the host.  --all adds the GEMM
kernel time of the other configurations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
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


GEMM_SOURCES = ["block_scaled_precision_act_amd/csrc/gemm_bf16.hip",
                "block_scaled_precision_act_amd/csrc/mx_internal.h",
                "block_scaled_precision_act_amd/csrc/mx_epilogue.h",
                "block_scaled_precision_act_amd/csrc/mx_quant.h"]
ACT_QUANT_SOURCES = ["block_scaled_precision_act_amd/csrc/act_quant.hip",
                     "block_scaled_precision_act_amd/csrc/mx_philox.h",
                     "block_scaled_precision_act_amd/csrc/mx_quant.h"]
# act_quant_kernel<chunks per lane, output format, stochastic>: format 0 is E4M3, 4 packed E2M1
AQ_E4M3_KERNEL = r"act_quant_kernel<\d+, 0, false>"
AQ_E2M1_KERNEL = r"act_quant_kernel<\d+, 4, false>"
# gemm_bf16_kernel<A format, B format, bias, quantized output, epilogue, split-K, BM, BN, ...>:
# format 0 is E4M3, 4 packed E2M1
GEMM_FP8_FP4_KERNEL = r"gemm_bf16_kernel<0, 4, true, false, 0, false, 256, 256,"
GEMM_FP8_FP4_QUANT_KERNEL = r"gemm_bf16_kernel<0, 4, true, true, 0, false, 256, 256,"
GEMM_FP8_FP4_128_KERNEL = r"gemm_bf16_kernel<0, 4, true, false, 0, false, 128, 128,"
GEMM_FP8_FP4_SPLITK_KERNEL = r"gemm_bf16_kernel<0, 4, true, false, 0, true, 256, 256,"
KERNEL_PATTERNS = (AQ_E4M3_KERNEL, AQ_E2M1_KERNEL, GEMM_FP8_FP4_KERNEL, GEMM_FP8_FP4_QUANT_KERNEL,
                   GEMM_FP8_FP4_128_KERNEL, GEMM_FP8_FP4_SPLITK_KERNEL)
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


def time_events(fn, iters, torch):
    """Average time per fn() over iters back-to-back calls: one pair of HIP events on the current
    stream (the stream every launch here goes to) brackets the whole run, so the figure is the
    kernels' own time plus the short gaps between back-to-back dispatches, not the longer gap an
    event marker between two kernels adds."""
    s = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(s)
    for _ in range(iters):
        fn()
    end.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters   # ms


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
    runs, total = 0, 0.0
    while runs < max_runs and (runs == 0 or total < min_seconds):
        t0 = time.perf_counter()
        codes, sb = O.act_quant(w.x[:rows])
        A = O.decode_e4m3_rows(codes, sb)
        B = O.decode_fp4_rows(w.b, w.b_s)
        ref, S = O.gemm_ref(A, B, O.bf16_to_f64(w.bias))
        total += time.perf_counter() - t0
        runs += 1
        del codes, sb, A, B, ref, S
    dt = total / runs
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3), "runs": runs,
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
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--aq-iters", type=int, default=50)
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
    stream = torch.cuda.current_stream()

    def step():
        mx.mx_act_quant(x, q, s, stream=stream)
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # the dominant kernel alone: the step's GEMM launched back to back on the same stream and
    # inputs, as many times as there are steps
    def gemm():
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias, stream=stream)

    gemm_ms = time_events(gemm, args.steps, torch)
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(gemm_tflops / MFMA_PEAK_TFLOPS["bf16"], 4),
                "traffic": _traffic("gemm_fp8_fp4_4096x7168x2048", GEMM_SOURCES),
                "mfma_util": _mfma_util("gemm_fp8_fp4_4096x7168x2048", GEMM_SOURCES),
                "kernel": "gemm_bf16_kernel<fp8, fp4, bias> (E4M3/E2M1 decoded exactly to bf16, "
                          "bf16 MFMA)", "avg_launch_ms": round(gemm_ms, 5),
                "algorithmic_flops_per_launch": flops,
                "frac_of_fp8_peak": round(gemm_tflops / MFMA_PEAK_TFLOPS["fp8"], 4),
                "peak_note": "peak is the bf16 MFMA's, the instruction this GEMM runs on: the FP8 "
                             "MFMA (5.0 PF) adds mixed-exponent products inexactly and misses the "
                             "2^-20*sum|a*b| bound; frac_of_fp8_peak is against the FP8 peak"}

    # ---- the same GEMM emitting the next layer's activation operand (E4M3 codes + per-32 E8M0
    # bytes of the bf16 output): the quantizing epilogue against the bf16 output followed by
    # act_quant on it, on the step's inputs.
    qn = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    qsn = torch.empty((M, N // 32), dtype=torch.uint8, device="cuda")

    def fused():
        mx.mx_gemm_fp8_fp4_quant(q, s, b, b_s, qn, qsn, bias=bias, stream=stream)

    def unfused():
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias, stream=stream)
        mx.mx_act_quant(c, qn, qsn, stream=stream)

    for _ in range(5):
        fused()
        unfused()
    fused_ms = time_events(fused, 50, torch)
    unfused_ms = time_events(unfused, 50, torch)
    next_layer = {"workload": "FP8xMXFP4 GEMM 4096x7168x2048 + bias -> E4M3 [4096, 7168] + "
                              "E8M0 [4096, 224] for the next layer",
                  "fused_ms": round(fused_ms, 5), "unfused_ms": round(unfused_ms, 5),
                  "fused_tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
                  "speedup": round(unfused_ms / fused_ms, 3),
                  "fused_traffic": _traffic("gemm_fp8_fp4_quant_4096x7168x2048", GEMM_SOURCES)}
    del qn, qsn

    # ---- the residual and GELU epilogues on the same GEMM (bf16 out), against the plain bias one
    res_t = torch.empty((M, N), dtype=torch.bfloat16, device="cuda").normal_()

    def with_residual():
        mx.mx_gemm_fp8_fp4_bias_residual(q, s, b, b_s, res_t, c, bias=bias, stream=stream)

    def with_gelu():
        mx.mx_gemm_fp8_fp4_bias_gelu(q, s, b, b_s, c, bias=bias, stream=stream)

    for _ in range(5):
        with_residual()
        with_gelu()
    res_ms = time_events(with_residual, 50, torch)
    gelu_ms = time_events(with_gelu, 50, torch)
    epilogues = {"workload": "FP8xMXFP4 GEMM 4096x7168x2048 + bias, bf16 out: + bf16 residual "
                             "[4096, 7168], or GELU",
                 "bias_ms": round(gemm_ms, 5),
                 "bias_residual_ms": round(res_ms, 5),
                 "bias_residual_tflops": round(flops / (res_ms * 1e-3) / 1e12, 2),
                 "bias_gelu_ms": round(gelu_ms, 5),
                 "bias_gelu_tflops": round(flops / (gelu_ms * 1e-3) / 1e12, 2)}
    del res_t

    # ---- split-K on the down-projection shape 4096x2048x7168 (128 output tiles of 256x256 for
    # 256 CUs): the same inputs through the plain and the split-K entry point
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

    for _ in range(200):
        down_plain()
        down_split()
    dflops = 2.0 * wd.M * wd.N * wd.K
    plain_ms = time_events(down_plain, 50, torch)
    split_ms = time_events(down_split, 50, torch)
    splitk = {"workload": "FP8xMXFP4 GEMM 4096x2048x7168 + bias (128 tiles of 256x256): plain "
                          "launch (128x128 tiles) against K split in two",
              "plain_ms": round(plain_ms, 5), "plain_tflops": round(dflops / (plain_ms * 1e-3) / 1e12, 2),
              "splitk_ms": round(split_ms, 5), "splitk_tflops": round(dflops / (split_ms * 1e-3) / 1e12, 2),
              "speedup": round(plain_ms / split_ms, 3), "workspace_bytes": int(wsd.numel())}
    del ad, asd, bd, bsd, biasd, cd, wsd

    # ---- the backward of the same linear layer y = x W^T (x [4096, 2048], W [7168, 2048],
    # dY [4096, 7168]): dX = dY W and dW = dY^T x from stochastically rounded E5M2 gradients and
    # transposed E4M3 operands, six kernels on one stream
    backward = bench_backward(mx, synth, torch, dev_bf16, w.x, stream)

    # ---- standalone act_quant on [16384, 7168], sustained: back-to-back launches rotating over
    # three input/output sets (1.07 GB, far beyond the 256 MB last-level cache), so each launch
    # reads its input from HBM and pays for the previous launch's write-back.
    xs_bits = synth.act_quant_standalone_16384x7168()
    xs = [dev_bf16(xs_bits)]
    del xs_bits
    xs += [xs[0].clone() for _ in range(2)]
    qs = [torch.empty(xs[0].shape, dtype=torch.uint8, device="cuda") for _ in range(3)]
    ss = [torch.empty((xs[0].shape[0], xs[0].shape[1] // 32), dtype=torch.uint8, device="cuda")
          for _ in range(3)]
    for i in range(6):
        mx.mx_act_quant(xs[i % 3], qs[i % 3], ss[i % 3], stream=stream)
    rot = [0]

    def aq_launch():
        i = rot[0] % 3
        rot[0] += 1
        mx.mx_act_quant(xs[i], qs[i], ss[i], stream=stream)

    aq_ms = time_events(aq_launch, args.aq_iters, torch)
    aq_bytes = ACT_QUANT_BYTES_PER_ELEM * xs[0].numel()
    aq_gbs = aq_bytes / (aq_ms * 1e-3) / 1e9
    act_quant = {"workload": "act_quant bf16 [16384, 7168] -> E4M3 + E8M0 (3 rotating buffer sets)",
                 "value": round(aq_gbs, 1), "unit": "GB/s", "avg_launch_ms": round(aq_ms, 5),
                 "roofline": {"bound": "hbm", "achieved": round(aq_gbs, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(aq_gbs / HBM_PEAK_GBS, 4),
                              "traffic": _traffic("act_quant_16384x7168", ACT_QUANT_SOURCES),
                              "algorithmic_bytes_per_launch": aq_bytes}}
    del qs

    # ---- the MXFP4 producer on the same three input sets (packed E2M1 out, [16384, 3584])
    q4 = [torch.empty((xs[0].shape[0], xs[0].shape[1] // 2), dtype=torch.uint8, device="cuda")
          for _ in range(3)]
    for i in range(6):
        mx.mx_act_quant_fp4(xs[i % 3], q4[i % 3], ss[i % 3], stream=stream)

    def aq4_launch():
        i = rot[0] % 3
        rot[0] += 1
        mx.mx_act_quant_fp4(xs[i], q4[i], ss[i], stream=stream)

    aq4_ms = time_events(aq4_launch, args.aq_iters, torch)
    aq4_bytes = ACT_QUANT_FP4_BYTES_PER_ELEM * xs[0].numel()
    aq4_gbs = aq4_bytes / (aq4_ms * 1e-3) / 1e9
    act_quant_fp4 = {"workload": "act_quant_fp4 bf16 [16384, 7168] -> packed E2M1 + E8M0 "
                                 "(3 rotating buffer sets)",
                     "value": round(aq4_gbs, 1), "unit": "GB/s", "avg_launch_ms": round(aq4_ms, 5),
                     "roofline": {"bound": "hbm", "achieved": round(aq4_gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(aq4_gbs / HBM_PEAK_GBS, 4),
                                  "traffic": _traffic("act_quant_fp4_16384x7168", ACT_QUANT_SOURCES),
                                  "algorithmic_bytes_per_launch": aq4_bytes}}
    del xs, q4, ss

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    others = None
    if args.all:
        others = bench_others(mx, synth, torch, dev_u8, dev_bf16, stream)

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "e4m3xe2m1->bf16 mfma, f32 acc",
           "data": "synthetic (seeded numpy PCG64; no dataset)",
           "config": {"workload": "act_quant x[4096,2048] -> FP8xMXFP4 GEMM 4096x7168x2048 + bias",
                      "M": M, "N": N, "K": K, "x_outliers": "1% x100",
                      "weight_scales": "E8M0 118..136", "parallelism": "single GPU"},
           "roofline": roofline, "act_quant": act_quant, "act_quant_fp4": act_quant_fp4,
           "gemm_only_tflops": round(gemm_tflops, 2)}
    out["next_layer_quant"] = next_layer
    out["epilogues"] = epilogues
    out["splitk"] = splitk
    out["backward"] = backward
    if others is not None:
        out["other_configs"] = others
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


def bench_backward(mx, synth, torch, dev_bf16, x_bits, stream):
    """dX and dW of the 4096x7168x2048 linear layer: each kernel over 50 back-to-back launches,
    then the whole six-kernel backward step."""
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

    for _ in range(100):
        step()
    res = {"workload": "backward of y = x W^T, x [4096, 2048], W [7168, 2048], dY [4096, 7168]: "
                       "dX = dY W (K split), dW = dY^T x; stochastic E5M2 gradients"}
    qbytes = {"quant_e5m2_dY": M * N, "quant_transpose_e4m3_W": N * K,
              "quant_transpose_e5m2_dY": M * N, "quant_transpose_e4m3_x": M * K}
    flops = 2.0 * M * N * K
    for name, f in steps.items():
        ms = time_events(f, 50, torch)
        entry = {"ms": round(ms, 5)}
        if name in qbytes:
            entry["gbs"] = round(ACT_QUANT_BYTES_PER_ELEM * qbytes[name] / (ms * 1e-3) / 1e9, 1)
        else:
            entry["tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
        res[name] = entry
    rne_ms = time_events(lambda: mx.mx_quant_e5m2(dY, gq, gs, stream=stream), 50, torch)
    res["quant_e5m2_dY_round_to_nearest"] = {
        "ms": round(rne_ms, 5), "gbs": round(ACT_QUANT_BYTES_PER_ELEM * M * N / (rne_ms * 1e-3) / 1e9, 1)}
    step_ms = time_events(step, 20, torch)
    res["step_ms"] = round(step_ms, 5)
    res["step_tflops"] = round(2 * flops / (step_ms * 1e-3) / 1e12, 2)
    return res


def bench_others(mx, synth, torch, dev_u8, dev_bf16, stream):
    """GEMM kernel time of the other configurations (operands already quantized in HBM).

    For each: `ms` over back-to-back launches on the stream (one event pair around the run).
    The latency-bound ones (the 16x256x512 and 1024^3 configurations and the A4W4 shapes) also
    report `graph_ms`, the time per launch of 20 launches captured in one HIP graph and replayed
    (launch overhead amortized), and `cold_ms`, the median time of single launches each after
    512 MB were written to evict the caches (events around the GEMM alone).  The A4W4 shapes
    also time their residual and GELU epilogues, and bias + GELU written as packed MXFP4 for the
    next A4W4 layer, fused and as GELU then the MXFP4 producer."""
    res = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

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

    def cold_ms(launch, iters=10):
        cur = torch.cuda.current_stream()
        ts = []
        for i in range(iters):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            launch(stream)
            b.record(cur)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    def run(w, kind, bias=True, latency=False, epilogues=False):
        if w.a_kind == "acts":
            xq = dev_bf16(w.x)
            shape = xq.shape
            a = torch.empty(shape, dtype=torch.uint8, device="cuda")
            a_s = torch.empty(shape[:-1] + (shape[-1] // 32,), dtype=torch.uint8, device="cuda")
            if xq.dim() == 3:
                mx.mx_act_quant_strided_batched(xq, a, a_s, stream=stream)
            else:
                mx.mx_act_quant(xq, a, a_s, stream=stream)
            del xq
        else:
            a, a_s = dev_u8(w.a), dev_u8(w.a_s)
        b, b_s = dev_u8(w.b), dev_u8(w.b_s)
        bias_t = dev_bf16(w.bias) if (bias and w.bias is not None) else None
        shape = (w.M, w.N) if w.batch is None else (w.batch, w.M, w.N)
        c = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        fn = getattr(mx, f"mx_gemm_{kind}")

        def launch(st):
            fn(a, a_s, b, b_s, c, bias=bias_t, stream=st)

        # warm up for about 50 ms of launches (past the clock drop sustained load brings)
        rough = time_events(lambda: launch(stream), 3, torch)
        for _ in range(max(3, int(50.0 / max(rough, 1e-3)))):
            launch(stream)
        ms = time_events(lambda: launch(stream), 20, torch)
        flops = 2.0 * w.M * w.N * w.K * (w.batch or 1)
        r = {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        if latency:
            r["graph_ms"] = round(graph_ms(launch), 5)
            r["cold_ms"] = round(cold_ms(launch), 5)
        if epilogues:
            resid = torch.empty(shape, dtype=torch.bfloat16, device="cuda").normal_()
            fr = getattr(mx, f"mx_gemm_{kind}_bias_residual")
            fg = getattr(mx, f"mx_gemm_{kind}_bias_gelu")
            for _ in range(3):
                fr(a, a_s, b, b_s, resid, c, bias=bias_t, stream=stream)
                fg(a, a_s, b, b_s, c, bias=bias_t, stream=stream)
            r["bias_residual_ms"] = round(time_events(
                lambda: fr(a, a_s, b, b_s, resid, c, bias=bias_t, stream=stream), 20, torch), 5)
            r["bias_gelu_ms"] = round(time_events(
                lambda: fg(a, a_s, b, b_s, c, bias=bias_t, stream=stream), 20, torch), 5)
            # the next A4W4 layer's operand straight from the epilogue, against GELU in bf16 then
            # the MXFP4 producer on it
            q = torch.empty(shape[:-1] + (w.N // 2,), dtype=torch.uint8, device="cuda")
            qs = torch.empty(shape[:-1] + (w.N // 32,), dtype=torch.uint8, device="cuda")
            fq = getattr(mx, f"mx_gemm_{kind}_bias_gelu_quant")

            def unfused():
                fg(a, a_s, b, b_s, c, bias=bias_t, stream=stream)
                mx.mx_act_quant_fp4(c, q, qs, stream=stream)

            for _ in range(3):
                fq(a, a_s, b, b_s, q, qs, bias=bias_t, stream=stream)
                unfused()
            r["bias_gelu_quant_ms"] = round(time_events(
                lambda: fq(a, a_s, b, b_s, q, qs, bias=bias_t, stream=stream), 20, torch), 5)
            r["bias_gelu_then_quant_ms"] = round(time_events(unfused, 20, torch), 5)
        return r

    res["fp8xmxfp4_16x256x512"] = run(synth.fp8xmxfp4_16x256x512(), "fp8_fp4", latency=True)
    res["fp8xfp8_1024^3_bias"] = run(synth.fp8xfp8_1024cubed_bias(), "fp8_fp8", latency=True)
    for i in range(3):
        w = synth.a4w4_skinny(i)
        r = run(w, "fp4_fp4", latency=True, epilogues=True)
        nbytes = w.M * w.K / 2 + w.M * w.K / 32 + w.N * w.K / 2 + w.N * w.K / 32 + 2 * w.M * w.N
        r["gbs"] = round(nbytes / (r["ms"] * 1e-3) / 1e9, 1)
        r["graph_gbs"] = round(nbytes / (r["graph_ms"] * 1e-3) / 1e9, 1)
        res[w.name] = r
    res["fp8xfp8_8x1024x2048x2048"] = run(synth.fp8xfp8_batched_8x1024x2048x2048(), "fp8_fp8")
    res["fp8xfp8_8192^3"] = run(synth.fp8xfp8_8192cubed(), "fp8_fp8")
    del flush
    return res


def _timed_region_averages(stats_dir):
    """Average kernel-trace duration of the dispatches inside each timed region of a default
    bench.py run (dispatch order = launch order on the one stream), with the HIP-event average
    the same run printed for that region."""
    import csv
    import glob
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return {}
    seq = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                seq.append((int(r["Start_Timestamp"]), r["Kernel_Name"],
                            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                            int(r["Grid_Size_X"])))
    seq.sort()
    line = {}
    out_txt = os.path.join(stats_dir, "bench_stdout.txt")
    if os.path.exists(out_txt):
        with open(out_txt) as fh:
            js = [ln for ln in fh if ln.startswith("{")]
        if js:
            line = json.loads(js[-1])
    steps, warmup = line.get("steps", 100), line.get("warmup", 200)

    def durs(pattern, grid=None):
        return [d / 1000.0 for _, k, d, g in seq
                if re.search(pattern, k) and (grid is None or g == grid)]

    res = {}
    # the GEMM's dispatches: warm-up steps, timed steps, then the back-to-back GEMM loop
    gall = durs(GEMM_FP8_FP4_KERNEL)
    g = gall[warmup + steps:warmup + 2 * steps]
    ev = line.get("roofline", {}).get("avg_launch_ms")
    if g:
        res["gemm_fp8_fp4 (back-to-back loop)"] = (len(g), sum(g) / len(g), ev and ev * 1e3)
    g = gall[warmup:warmup + steps]
    if g:
        res["gemm_fp8_fp4 (inside the timed steps)"] = (len(g), sum(g) / len(g), None)
    big = max((gr for _, k, _, gr in seq if re.search(AQ_E4M3_KERNEL, k)), default=None)
    a8 = durs(AQ_E4M3_KERNEL, big)[6:]
    ev = line.get("act_quant", {}).get("avg_launch_ms")
    if a8:
        res["act_quant [16384, 7168]"] = (len(a8), sum(a8) / len(a8), ev and ev * 1e3)
    a4 = durs(AQ_E2M1_KERNEL)[6:]
    ev = line.get("act_quant_fp4", {}).get("avg_launch_ms")
    if a4:
        res["act_quant_fp4 [16384, 7168]"] = (len(a4), sum(a4) / len(a4), ev and ev * 1e3)
    q = durs(GEMM_FP8_FP4_QUANT_KERNEL)[5:]
    ev = line.get("next_layer_quant", {}).get("fused_ms")
    if q:
        res["gemm_fp8_fp4_quant (fused next layer)"] = (len(q), sum(q) / len(q), ev and ev * 1e3)
    return res


def summarize(stats_dir, fetch_dir, write_dir):
    """Writes the profiles/ summaries from rocprofv3 CSV output of this script:
    kernel-trace stats, and FETCH_SIZE / WRITE_SIZE per dispatch scaled by what the same counters
    read for the plain 1 GiB copy (--copy-calibration)."""
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
    aq_alg = ACT_QUANT_BYTES_PER_ELEM * 16384 * 7168
    aq4_alg = ACT_QUANT_FP4_BYTES_PER_ELEM * 16384 * 7168
    gemm_in = 4096 * 2048 + 4096 * 64 + 7168 * 1024 + 7168 * 64 + 2 * 7168
    gemm_alg = gemm_in + 2 * 4096 * 7168
    gemm_q_alg = gemm_in + 4096 * 7168 + 4096 * 7168 // 32
    # the split-K line's down-projection 4096x2048x7168 (its partial tiles are not algorithmic)
    down_alg = 4096 * 7168 + 4096 * 224 + 2048 * 3584 + 2048 * 224 + 2 * 2048 + 2 * 4096 * 2048
    out = {}
    for name, part, grid, files, alg in (
            ("act_quant_16384x7168", aq8, aq_grid, ACT_QUANT_SOURCES, aq_alg),
            ("act_quant_fp4_16384x7168", aq4, None, ACT_QUANT_SOURCES, aq4_alg),
            ("gemm_fp8_fp4_4096x7168x2048", GEMM_FP8_FP4_KERNEL, None,
             GEMM_SOURCES, gemm_alg),
            ("gemm_fp8_fp4_quant_4096x7168x2048", GEMM_FP8_FP4_QUANT_KERNEL, None,
             GEMM_SOURCES, gemm_q_alg),
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
    timed = _timed_region_averages(stats_dir)
    cmds = {
        "stats": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/stats -o run "
                 "-- python3 bench.py --no-cpu > OUT/stats/bench_stdout.txt",
        "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run "
                 "-- python3 bench.py --steps 2 --warmup 1 --no-cpu --aq-iters 2 --copy-calibration",
        "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run "
                 "-- python3 bench.py --steps 2 --warmup 1 --no-cpu --aq-iters 2 --copy-calibration",
        "summary": "python bench.py --summarize OUT/stats OUT/fetch OUT/write",
    }
    lines = ["rocprofv3 kernel-trace statistics of one bench.py run at its default settings",
             "(act_quant x[4096,2048] -> FP8xMXFP4 GEMM 4096x7168x2048 + bias, 200 warm-up and 100",
             "timed steps, then 100 back-to-back launches of the GEMM alone; the fused next-layer",
             "GEMM and the unfused GEMM + act_quant, 5 warm-up and 50 timed each; 6 warm-up and 50",
             "timed standalone act_quant launches on x[16384,7168], and as many of the MXFP4",
             "producer act_quant_fp4).", "",
             "command: " + cmds["stats"],
             "(TMPDIR=/tmp, repository root as cwd, OUT the folder the profiler writes to)", ""]
    if stats:
        keys = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "StdDev", "Percentage"]
        lines.append(" | ".join(keys))
        for r in stats:
            lines.append(" | ".join(str(r.get(k, "")) for k in keys))
    if timed:
        lines += ["", "Timed-region dispatches only, from the kernel trace of the same run, beside",
                  "the HIP-event average that run's bench.py line reports for them:"]
        for name, (n, trace_us, event_us) in timed.items():
            ev = "n/a" if event_us is None else f"{event_us:.2f} us"
            lines.append(f"  {name}: {n} dispatches, trace average {trace_us:.2f} us, "
                         f"events {ev}")
    with open(os.path.join(prof, "kernel_stats_act_quant_and_gemm_fp8_fp4_4096x7168x2048.txt"), "w") as fh:
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
    with open(os.path.join(prof, "traffic_act_quant_16384x7168_and_gemm_fp8_fp4_4096x7168x2048.txt"), "w") as fh:
        fh.write("\n".join(tl) + "\n")
    print("\n".join(lines + [""] + tl))


BUSY_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE "
                 "SQ_INSTS_MFMA")


def summarize_busy(busy_dir, prof_dir=None):
    """MFMA utilisation of the 4096x7168x2048 GEMM from one rocprofv3 --pmc run of BUSY_COUNTERS
    with --kernel-trace (the trace gives each dispatch's duration).  Counter values in the csv are
    sums over the XCDs and shader engines.  Per dispatch:
    * active cycles g = GRBM_GUI_ACTIVE / XCDs (the GUI counter runs once per XCD), clock = g / ns;
    * mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (g * SIMDs), rocprofv3's own MfmaUtil;
    * cu_busy = SQ_BUSY_CU_CYCLES / (g * CUs), and mfma_busy_over_busy_cu = MFMA-busy cycles over
      the SIMD cycles of CUs that hold a workgroup.  SQ_BUSY_CU_CYCLES is read in plain cycles:
      read as quad-cycles it would exceed CUs * g threefold.
    Medians over the dispatches are written to mfma_util_<kernel>.json and .txt in prof_dir
    (profiles/ by default) and returned."""
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
    ctr = {}
    for r in rows("*counter_collection.csv"):
        if re.search(GEMM_FP8_FP4_KERNEL, r["Kernel_Name"]):
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
                    "mfma_busy_cycles_per_inst": v["SQ_VALU_MFMA_BUSY_CYCLES"] / v["SQ_INSTS_MFMA"]})
    if not per:
        print("no GEMM dispatches with every counter found", file=sys.stderr)
        return None
    med = {k: round(statistics.median(d[k] for d in per), 4) for k in per[0]}
    M, N, K = 4096, 7168, 2048
    cmd = (f"rocprofv3 --pmc {BUSY_COUNTERS} --kernel-trace --output-format csv -d OUT/busy -o run "
           "-- python3 bench.py --steps 2 --warmup 1 --no-cpu --aq-iters 2")
    out = {"source_hash": _kernel_hash(GEMM_SOURCES), "dispatches": len(per),
           "simds": simds, "cus": cus, "xcds": xcds,
           "mfma_insts_expected": 2 * M * N * K // (32 * 32 * 16 * 2), **med, "command": cmd}
    prof = prof_dir or os.path.join(HERE, "profiles")
    name = "mfma_util_gemm_fp8_fp4_4096x7168x2048"
    with open(os.path.join(prof, name + ".json"), "w") as fh:
        json.dump(out, fh, indent=1)
    txt = [f"MFMA utilisation of the FP8xMXFP4 GEMM 4096x7168x2048 + bias (bf16 MFMA 32x32x16),",
           f"medians over {len(per)} dispatches of one counter run:", "",
           "command (TMPDIR=/tmp, repository root as cwd, OUT the folder the profiler writes to):",
           "  " + cmd, "  python bench.py --summarize-busy OUT/busy", "",
           f"duration {med['duration_us']} us at {med['clock_ghz']} GHz "
           f"(GRBM_GUI_ACTIVE over the {xcds} XCDs / duration)",
           f"MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x {simds} SIMDs) = {med['mfma_util']}",
           f"CUs holding a workgroup: {med['cu_busy']} of the active cycles; MFMA-busy over their "
           f"SIMD cycles = {med['mfma_busy_over_busy_cu']}",
           f"MFMA instructions {med['mfma_insts']:.0f} (2MNK/32768 = {out['mfma_insts_expected']}), "
           f"{med['mfma_busy_cycles_per_inst']} busy cycles each",
           f"source hash {out['source_hash']}"]
    with open(os.path.join(prof, name + ".txt"), "w") as fh:
        fh.write("\n".join(txt) + "\n")
    print("\n".join(txt))
    return out


if __name__ == "__main__":
    main()
