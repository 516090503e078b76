"""The per-matrix size limit (just under 2^31 elements) on the GPU: every index past 2^31 bytes
or elements must be computed in 64 bits.  Inputs are drawn on the GPU (seeded); sampled rows,
the last ones included, are copied back and checked against the oracle.  A size one element
over the limit is refused on the host (tested without a GPU in test_abi)."""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import host_bf16_bits, host_u8, note

pytestmark = pytest.mark.gpu

M_MAX, K_MAX = 65535, 32768           # 2^31 - 32768 elements: the largest M at this K


def _rows(M, n=48, seed=0):
    r = np.random.default_rng(seed).integers(0, M, n)
    return np.unique(np.concatenate([r, [0, M // 2, M - 2, M - 1]]))


def test_act_quant_at_the_size_limit(mx):
    note(f"act_quant {M_MAX}x{K_MAX}")
    x = synth.bf16_normal_device(9001, (M_MAX, K_MAX))
    q = torch.empty((M_MAX, K_MAX), dtype=torch.uint8, device="cuda")
    s = torch.empty((M_MAX, K_MAX // 32), dtype=torch.uint8, device="cuda")
    mx.mx_act_quant(x, q, s)
    torch.cuda.synchronize()
    rows = _rows(M_MAX)
    xr = host_bf16_bits(x[torch.from_numpy(rows).cuda()])
    rq, rs = O.act_quant(xr)
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(host_u8(q[idx]), rq) and np.array_equal(host_u8(s[idx]), rs)
    del x, q, s


def test_e5m2_quant_at_the_size_limit(mx):
    note(f"quant_e5m2 stochastic {M_MAX}x{K_MAX}")
    x = synth.bf16_normal_device(9002, (M_MAX, K_MAX), std=1e-3)
    q = torch.empty((M_MAX, K_MAX), dtype=torch.uint8, device="cuda")
    s = torch.empty((M_MAX, K_MAX // 32), dtype=torch.uint8, device="cuda")
    mx.mx_quant_e5m2(x, q, s, seed=77)
    torch.cuda.synchronize()
    rows = _rows(M_MAX, seed=1)
    idx = torch.from_numpy(rows).cuda()
    xr = host_bf16_bits(x[idx])
    # the draw index of a row is its position in the whole output: check the rows one by one
    sb = O.grad_scale_bytes(xr)
    assert np.array_equal(host_u8(s[idx]), sb)
    y = (O.bf16_to_f64(xr).reshape(len(rows), -1, 32) / O.e8m0_to_f64(sb)[..., None]).reshape(len(rows), -1)
    base = rows.astype(np.uint64)[:, None] * np.uint64(K_MAX) + np.arange(K_MAX, dtype=np.uint64)[None, :]
    u = O.uniform_u32(77, base)
    assert np.array_equal(host_u8(q[idx]), O.e5m2_encode_stochastic(y, u))
    del x, q, s


def test_quant_transpose_at_the_size_limit(mx):
    R, C = 65504, 32768                  # R % 32 == 0, R * C < 2^31
    note(f"quant_transpose_e4m3 {R}x{C}")
    x = synth.bf16_normal_device(9003, (R, C))
    q = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    s = torch.empty((C, R // 32), dtype=torch.uint8, device="cuda")
    mx.mx_quant_transpose_e4m3(x, q, s)
    torch.cuda.synchronize()
    cols = _rows(C, seed=2)                                  # output rows = input columns
    idx = torch.from_numpy(cols).cuda()
    xc = host_bf16_bits(x[:, idx].t().contiguous())        # [len(cols), R]
    rq, rs = O.act_quant(xc)
    assert np.array_equal(host_u8(q[idx]), rq) and np.array_equal(host_u8(s[idx]), rs)
    del x, q, s


def test_gemm_with_a_at_the_size_limit(mx):
    N = 256
    note(f"gemm fp8_fp4 {M_MAX}x{N}x{K_MAX}")
    a = synth.e4m3_uniform_nonnan_device(9004, (M_MAX, K_MAX))
    a_s = synth.e8m0_uniform_device(9005, (M_MAX, K_MAX // 32))
    rng = synth.rng_for(9006)
    b = synth.fp4_packed_uniform(rng, N, K_MAX)
    b_s = synth.e8m0_uniform(rng, (N, K_MAX // 32))
    bias = synth.bf16_normal(rng, (N,), std=0.1)
    c = torch.full((M_MAX, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    from gpu_util import dev_bf16, dev_u8
    mx.mx_gemm_fp8_fp4(a, a_s, dev_u8(b), dev_u8(b_s), c, bias=dev_bf16(bias))
    torch.cuda.synchronize()
    rows = _rows(M_MAX, n=24, seed=3)
    idx = torch.from_numpy(rows).cuda()
    A = O.decode_e4m3_rows(host_u8(a[idx]), host_u8(a_s[idx]))
    ref, S = O.gemm_ref(A, O.decode_fp4_rows(b, b_s), O.bf16_to_f64(bias))
    out = host_bf16_bits(c[idx])
    assert O.within_tolerance(out, ref, S).all()
    assert np.isfinite(O.bf16_to_f64(host_bf16_bits(c[-256:]))).all()
    del a, a_s, c
