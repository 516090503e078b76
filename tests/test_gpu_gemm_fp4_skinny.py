"""The skinny MXFP4 x MXFP4 GEMM (M <= 64) whose codes are staged through LDS (K % 256 == 0),
against the oracle.

Every case is a shape that takes that kernel: M <= 64 and K % 256 == 0.  Its three launch forms
are all covered: one 2-step chunk per wavefront with 4 wavefronts (up to 8 steps of K) or 6 (up
to 12), and the two-buffer ring of 8 wavefronts (or 4 when 64 rows and 32 columns would not fit)
for longer K, whose wavefronts each take several chunks; 16-column workgroups, and 32-column ones
where the 16-column grid would not fit in one wave of the CUs; and, where twice the 16-column
grid fits in one wave (and M > 16), two workgroups per column block with half the row tiles each
(the second one's last tile partly or wholly past M).  Ragged M (every tile count 1-4,
rows past M in the last tile) and N (columns past N in the last workgroup), batches, the bias, the
residual and GELU epilogues, and the MXFP4-quantized output.  Each output is checked against
the float64 reference of the same bytes within |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k|
(the GELU and quantized outputs within the bounds their oracles derive).
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16
from test_gpu_gemm import assert_within, check_workload, operands
from test_gpu_gemm_quant_fp4 import _oracle_check, run_fused, run_unfused

pytestmark = pytest.mark.gpu


def takes_lds_kernel(M, K):
    return M <= 64 and K % 256 == 0


def wide_workgroups(N, batch=1, cus=256):
    """32 columns per workgroup: where 16-column workgroups would not fit in one wave."""
    return -(-N // 16) * batch > cus


def row_split(M, N, batch=1, cus=256):
    """Two workgroups per column block, half the row tiles each (the plain and epilogue forms)."""
    return M > 16 and 2 * -(-N // 16) * batch <= cus


def test_headline_rules():
    assert row_split(41, 1536) and not row_split(41, 4608) and wide_workgroups(4608)
    assert not row_split(16, 1000) and row_split(17, 33)


SHAPES = [(1, 1, 256), (16, 16, 512), (17, 33, 1024), (33, 200, 1536), (41, 4607, 1536),
          (48, 100, 768), (64, 130, 2048), (41, 96, 3072), (64, 64, 6144), (9, 1537, 6144),
          (41, 300, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_shapes_against_oracle(mx, M, N, K, with_bias):
    assert takes_lds_kernel(M, K)
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=M * 131 + N * 7 + K + with_bias,
                          with_bias=with_bias)
    check_workload(mx, w)


@pytest.mark.parametrize("M,N,K", [(41, 96, 1536), (20, 70, 4096), (20, 2000, 1024)])
def test_batched(mx, M, N, K):
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=M + N + K, batch=3, with_bias=True)
    check_workload(mx, w)


# 32-column workgroups (more 16-column workgroups than CUs): ragged N (a workgroup with 16 or
# fewer live columns), every tile count, one buffer and the ring
@pytest.mark.parametrize("M,N,K", [(41, 4608, 1536), (41, 6144, 1536), (41, 4100, 1536),
                                   (16, 4111, 512), (64, 5000, 1024), (33, 8192, 3072),
                                   (48, 4200, 6144)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_wide_workgroups(mx, M, N, K, with_bias):
    assert takes_lds_kernel(M, K) and wide_workgroups(N)
    check_workload(mx, synth.gemm_inputs("fp4", "fp4", M, N, K, seed=3 * M + N + K + with_bias,
                                         with_bias=with_bias))


@pytest.mark.parametrize("M,N,K", [(41, 4608, 1536), (41, 1536, 6144)])
def test_headline_shapes_take_it(mx, M, N, K):
    # the three A4W4 configurations' shapes (41, 4608 | 6144 | 1536, ...) all take this kernel
    assert takes_lds_kernel(M, K)
    check_workload(mx, synth.gemm_inputs("fp4", "fp4", M, N, K, seed=3 * M + N + K))


@pytest.mark.parametrize("epi", ["residual", "gelu"])
@pytest.mark.parametrize("M,N,K", [(41, 200, 1536), (64, 96, 6144), (41, 4100, 1536)])
def test_epilogues(mx, epi, M, N, K):
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=M + 5 * N + K, with_bias=True)
    a, a_s, _, A, B, bias = operands(w)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    c = poison_bf16((M, N))
    note(f"gemm fp4_fp4 {epi} {M}x{N}x{K} (LDS-staged skinny)")
    if epi == "residual":
        res = synth.bf16_normal(synth.rng_for(M + N), (M, N))
        mx.mx_gemm_fp4_fp4_bias_residual(*args, dev_bf16(res), c, bias=dev_bf16(w.bias))
    else:
        mx.mx_gemm_fp4_fp4_bias_gelu(*args, c, bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    if epi == "residual":
        ref, S = O.gemm_residual_ref(A, B, bias, res)
        assert_within(out, ref, S, "residual")
    else:
        _, pre, S = O.gemm_gelu_ref(A, B, bias)
        ok = O.gelu_within(out, pre, S)
        assert ok.all(), f"gelu: {np.count_nonzero(~ok)} of {ok.size} outside the bound"


@pytest.mark.parametrize("gelu", [False, True])
@pytest.mark.parametrize("M,N,K", [(41, 4608, 1536), (64, 320, 6144), (17, 64, 2048)])
def test_quantized_output(mx, gelu, M, N, K):
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=M + N + 11 * K + gelu, with_bias=True)
    a, a_s, _, A, B, bias = operands(w)
    note(f"gemm fp4_fp4 quant gelu={gelu} {M}x{N}x{K} (LDS-staged skinny)")
    q, qs = run_fused(mx, "fp4_fp4", gelu, a, a_s, w.b, w.b_s, w.bias, M, N)
    q2, qs2 = run_unfused(mx, "fp4_fp4", gelu, a, a_s, w.b, w.b_s, w.bias, M, N)
    assert np.array_equal(q, q2) and np.array_equal(qs, qs2)
    _oracle_check("fp4_fp4", gelu, q, qs, A, B, bias, f"{M}x{N}x{K}")


def test_zero_weight_gives_bias_bit_exact(mx):
    M, N, K = 41, 300, 1536
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=77, with_bias=True)
    b = np.zeros_like(w.b)
    c = poison_bf16((M, N))
    note("gemm fp4_fp4 zero weight (LDS-staged skinny)")
    mx.mx_gemm_fp4_fp4(dev_u8(w.a), dev_u8(w.a_s), dev_u8(b), dev_u8(w.b_s), c,
                       bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(c), np.broadcast_to(w.bias, (M, N)))
