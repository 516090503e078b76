"""Seeded synthetic inputs for the act_quant producer and the block-scaled GEMM.

This module only draws random bytes; it holds none of the quantization or GEMM arithmetic.
Every generator takes a numpy PCG64 Generator and returns raw patterns:

* bf16 activations: float32 normal draws, optionally with a fraction of entries multiplied by
  an outlier factor, rounded once to bf16 (round to nearest even) by torch's CPU cast, returned
  as uint16 bit patterns;
* E4M3 codes: uniform over the 254 bytes that are not NaN (0x7F and 0xFF are skipped);
* packed E2M1 bytes: uniform bytes (two independent uniform 4-bit codes per byte);
* E8M0 scale bytes: uniform integers in [lo, hi], both ends included.

The named workloads follow the five configurations of the method's headline measurement, one
seed each (1001..1005).

Inputs at the per-matrix size limit (2^31 elements) are drawn on the GPU instead, with torch's
seeded device generator, in row chunks (the *_device functions); their bytes are copied back
only for the rows a test checks.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_normal(rng: np.random.Generator, shape, std: float = 1.0,
                outlier_frac: float = 0.0, outlier_mult: float = 100.0) -> np.ndarray:
    """uint16 bf16 patterns of N(0, std^2) draws; each entry independently (probability
    ``outlier_frac``) multiplied by ``outlier_mult`` before the single bf16 rounding."""
    import torch
    f = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        f *= np.float32(std)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape, dtype=np.float32) < outlier_frac
        f[mask] *= np.float32(outlier_mult)
    t = torch.from_numpy(f).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _device_generator(seed: int):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def bf16_normal_device(seed: int, shape, std: float = 1.0, chunk_rows: int = 4096):
    """A cuda bfloat16 tensor of N(0, std^2) float32 draws rounded once to bf16, drawn on the GPU
    from torch's generator seeded with ``seed``, chunk_rows rows at a time."""
    import torch
    g = _device_generator(seed)
    rows, cols = shape
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r)
        f = torch.randn((n, cols), generator=g, device="cuda", dtype=torch.float32)
        out[r:r + n] = (f * std).to(torch.bfloat16)
    return out


def e4m3_uniform_nonnan_device(seed: int, shape, chunk_rows: int = 4096):
    """A cuda uint8 tensor uniform over the 254 non-NaN e4m3fn codes, drawn on the GPU."""
    import torch
    g = _device_generator(seed)
    rows, cols = shape
    out = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    for r in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r)
        v = torch.randint(0, 254, (n, cols), generator=g, device="cuda", dtype=torch.int32)
        out[r:r + n] = (v + (v >= 0x7F).to(torch.int32)).to(torch.uint8)
    return out


def e8m0_uniform_device(seed: int, shape, lo: int = 118, hi: int = 136):
    import torch
    g = _device_generator(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)


def e4m3_uniform_nonnan(rng: np.random.Generator, shape) -> np.ndarray:
    """Bytes uniform over the 254 non-NaN e4m3fn codes (0x7F and 0xFF never drawn)."""
    r = rng.integers(0, 254, size=shape, dtype=np.int64)
    r = r + (r >= 0x7F)            # 0..126 -> 0x00..0x7E ; 127..253 -> 0x80..0xFE
    return r.astype(np.uint8)


def fp4_packed_uniform(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """[rows, k/2] bytes, every 4-bit code uniform in 0..15."""
    return rng.integers(0, 256, size=(rows, k // 2), dtype=np.int64).astype(np.uint8)


def e8m0_uniform(rng: np.random.Generator, shape, lo: int = 118, hi: int = 136) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)


@dataclass
class GemmWorkload:
    """Bytes of one GEMM problem.  ``a_kind`` is "acts" (bf16 activations to be quantized per 32),
    "fp8" (E4M3 codes + per-row-32 scales) or "fp4" (packed E2M1 + per-row-32 scales);
    ``b_kind`` is "fp4" (packed E2M1 + per-row-32 scales) or "fp8" (E4M3 + 32x32 block scales).
    Arrays carry a leading batch dimension when ``batch`` is not None."""
    name: str
    a_kind: str
    b_kind: str
    M: int
    N: int
    K: int
    batch: int | None = None
    x: np.ndarray | None = None          # bf16 patterns [.., M, K]   (a_kind == "acts")
    a: np.ndarray | None = None          # codes [.., M, K] or packed [.., M, K/2]
    a_s: np.ndarray | None = None        # [.., M, K/32]
    b: np.ndarray | None = None          # [.., N, K] (fp8) or [.., N, K/2] (fp4)
    b_s: np.ndarray | None = None        # [.., N, K/32] (fp4) or [.., ceil(N/32), ceil(K/32)] (fp8)
    bias: np.ndarray | None = None       # bf16 patterns [.., N]
    meta: dict = field(default_factory=dict)


def gemm_inputs(a_kind: str, b_kind: str, M: int, N: int, K: int, seed: int, *,
                batch: int | None = None, with_bias: bool = False, bias_std: float = 0.1,
                outlier_frac: float = 0.0, scale_lo: int = 118, scale_hi: int = 136,
                name: str = "") -> GemmWorkload:
    """Draw every byte of one problem in a fixed order: A side, B side, bias."""
    rng = rng_for(seed)
    lead = () if batch is None else (batch,)
    w = GemmWorkload(name=name or f"{a_kind}x{b_kind}_m{M}_n{N}_k{K}", a_kind=a_kind,
                     b_kind=b_kind, M=M, N=N, K=K, batch=batch)
    kb = -(-K // 32)
    if a_kind == "acts":
        w.x = bf16_normal(rng, lead + (M, K), outlier_frac=outlier_frac)
    elif a_kind == "fp8":
        w.a = e4m3_uniform_nonnan(rng, lead + (M, K))
        w.a_s = e8m0_uniform(rng, lead + (M, kb), scale_lo, scale_hi)
    elif a_kind == "fp4":
        w.a = fp4_packed_uniform(rng, int(np.prod(lead + (M,))), K).reshape(lead + (M, K // 2))
        w.a_s = e8m0_uniform(rng, lead + (M, kb), scale_lo, scale_hi)
    else:
        raise ValueError(a_kind)
    if b_kind == "fp4":
        w.b = fp4_packed_uniform(rng, int(np.prod(lead + (N,))), K).reshape(lead + (N, K // 2))
        w.b_s = e8m0_uniform(rng, lead + (N, kb), scale_lo, scale_hi)
    elif b_kind == "fp8":
        w.b = e4m3_uniform_nonnan(rng, lead + (N, K))
        w.b_s = e8m0_uniform(rng, lead + (-(-N // 32), kb), scale_lo, scale_hi)
    else:
        raise ValueError(b_kind)
    if with_bias:
        w.bias = bf16_normal(rng, lead + (N,), std=bias_std)
    return w


# The five headline configurations (seeds 1001..1005).
def fp8xmxfp4_16x256x512() -> GemmWorkload:
    return gemm_inputs("acts", "fp4", 16, 256, 512, 1001, name="fp8xmxfp4_m16_n256_k512")


def fp8xfp8_1024cubed_bias() -> GemmWorkload:
    return gemm_inputs("acts", "fp8", 1024, 1024, 1024, 1002, with_bias=True,
                       name="fp8xfp8_m1024_n1024_k1024_bias")


SKINNY_A4W4_SHAPES = ((41, 4608, 1536), (41, 6144, 1536), (41, 1536, 6144))


def a4w4_skinny(i: int) -> GemmWorkload:
    M, N, K = SKINNY_A4W4_SHAPES[i]
    return gemm_inputs("fp4", "fp4", M, N, K, 1003 + 100 * i,
                       name=f"mxfp4xmxfp4_m{M}_n{N}_k{K}")


def fp8xfp8_8192cubed() -> GemmWorkload:
    return gemm_inputs("acts", "fp8", 8192, 8192, 8192, 1004, name="fp8xfp8_m8192_n8192_k8192")


def fp8xfp8_batched_8x1024x2048x2048() -> GemmWorkload:
    return gemm_inputs("acts", "fp8", 1024, 2048, 2048, 1104, batch=8,
                       name="fp8xfp8_b8_m1024_n2048_k2048")


def fp8xmxfp4_4096x7168x2048_bias() -> GemmWorkload:
    return gemm_inputs("acts", "fp4", 4096, 7168, 2048, 1005, with_bias=True, outlier_frac=0.01,
                       name="fp8xmxfp4_m4096_n7168_k2048_bias_outliers")


def act_quant_standalone_16384x7168() -> np.ndarray:
    """bf16 patterns [16384, 7168], N(0,1) with 1% of entries x100 before rounding."""
    return bf16_normal(rng_for(1205), (16384, 7168), outlier_frac=0.01)
