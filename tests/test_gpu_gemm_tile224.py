"""The 256 x 224 output tiles of the large-problem GEMM kernel against the oracle.

The library picks 256 x 224 tiles over 256 x 256 ones where they fill the CUs' waves better
(4096 x 7168: 448 tiles of 256 x 256 fill 1.75 waves of 256 CUs, 512 tiles of 256 x 224 fill two
waves exactly).  Every case here is a shape for which that choice is made (checked on the host
with the same rule, so that a change of the rule cannot silently take the tests off that path),
with ragged M and N edges, every operand kind and every epilogue, each output against the float64
reference from the same bytes within |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k|.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16
from test_gpu_gemm import assert_within, check_workload, operands

pytestmark = pytest.mark.gpu

CUS = 256


def picks_224(M, N, K, batch=1):
    """The library's rule for the large-problem kernel and its tile width, for one MI355X."""
    def tiles(bn):
        return -(-M // 256) * -(-N // bn) * batch
    large = 2 * tiles(256) > CUS and K % 512 == 0
    waves = lambda bn: -(-tiles(bn) // CUS)
    return large and waves(224) * 224 < waves(256) * 256


CASES = [("acts", "fp4", 2000, 7000, 512, None, True),     # ragged M (208) and N (56) edges
         ("acts", "fp8", 1800, 7168, 1024, None, False),
         ("acts", "fp8", 2048, 6999, 512, None, True),     # odd N: per-chunk copy-out
         ("fp4", "fp4", 2048, 7100, 512, None, True),
         ("fp8", "fp4", 1024, 7000, 512, 2, True)]         # batched: 2 x 128 tiles


@pytest.mark.parametrize("a_kind,b_kind,M,N,K,batch,with_bias", CASES)
def test_shapes_against_oracle(mx, a_kind, b_kind, M, N, K, batch, with_bias):
    assert picks_224(M, N, K, batch or 1)
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M + 3 * N + K, batch=batch,
                          with_bias=with_bias)
    check_workload(mx, w)


def test_headline_shape_takes_the_narrow_tiles():
    # 4096 x 7168 x 2048: the workload these tiles are for.
    assert picks_224(4096, 7168, 2048)
    # 8192^3 (1024 tiles of 256 x 256, four full waves) and the batched 8 x 1024 x 2048 (256
    # tiles, one full wave) keep the square tiles.
    assert not picks_224(8192, 8192, 8192)
    assert not picks_224(1024, 2048, 2048, 8)


@pytest.mark.parametrize("epi", ["residual", "gelu"])
def test_epilogues(mx, epi):
    M, N, K = 2000, 7000, 512
    assert picks_224(M, N, K)
    w = synth.gemm_inputs("acts", "fp4", M, N, K, seed=91, with_bias=True)
    a, a_s, _, A, B, bias = operands(w)
    kind = "fp8_fp4"
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    c = poison_bf16((M, N))
    note(f"gemm {kind} {epi} {M}x{N}x{K} (256x224 tiles)")
    if epi == "residual":
        res = synth.bf16_normal(synth.rng_for(92), (M, N))
        getattr(mx, f"mx_gemm_{kind}_bias_residual")(*args, dev_bf16(res), c, bias=dev_bf16(w.bias))
    else:
        getattr(mx, f"mx_gemm_{kind}_bias_gelu")(*args, c, bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    if epi == "residual":
        ref, S = O.gemm_residual_ref(A, B, bias, res)
        assert_within(out, ref, S, "residual")
    else:
        _, pre, S = O.gemm_gelu_ref(A, B, bias)
        ok = O.gelu_within(out, pre, S)
        assert ok.all(), f"gelu: {np.count_nonzero(~ok)} of {ok.size} outside the bound"


def test_quantized_output_matches_gemm_then_act_quant(mx):
    # The fused next-layer quantization on 256 x 224 tiles (N % 32 == 0) gives the bytes that the
    # bf16 GEMM followed by act_quant gives, and meets the bound against the oracle.
    M, N, K = 2000, 7168, 512
    assert picks_224(M, N, K)
    w = synth.gemm_inputs("acts", "fp4", M, N, K, seed=93, with_bias=True)
    a, a_s, _, A, B, bias = operands(w)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    q = torch.full((M, N), 0x7F, dtype=torch.uint8, device="cuda")
    qs = torch.full((M, N // 32), 0xFF, dtype=torch.uint8, device="cuda")
    note(f"gemm fp8_fp4 quant {M}x{N}x{K} (256x224 tiles)")
    mx.mx_gemm_fp8_fp4_quant(*args, q, qs, bias=dev_bf16(w.bias))
    c = poison_bf16((M, N))
    mx.mx_gemm_fp8_fp4(*args, c, bias=dev_bf16(w.bias))
    q2 = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    qs2 = torch.empty((M, N // 32), dtype=torch.uint8, device="cuda")
    mx.mx_act_quant(c, q2, qs2)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(qs, qs2)
    ref, S, _, _, _ = O.gemm_act_quant_ref(A, B, bias)
    ok = O.quant_output_within(q.cpu().numpy(), qs.cpu().numpy(), ref, S)
    assert ok.all(), f"{np.count_nonzero(~ok)} of {ok.size} outside the bound"
