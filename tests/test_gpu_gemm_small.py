"""The GEMM kernel for few output tiles and a short K (64x64 tiles, at most one per CU, the tile's
whole K copied into LDS at the start: K % 256 == 0, K <= 1024) against the oracle.

Every case is a shape that takes this kernel, checked on the host with the library's dispatch rule
(so a change of the rule cannot silently take the tests off it): every operand pairing, K of one
to four 256-wide chunks, ragged M and N, batches with distinct or shared operands, the bias,
residual and GELU epilogues, the quantized outputs (byte-equal to the bf16 GEMM followed by the
matching producer), and the E5M2 x E4M3 backward operands.  Outputs must meet
|out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k| against the float64 reference of the same bytes
(GELU and quantized outputs: the bounds their oracles derive).
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16
from test_gpu_gemm import assert_within, check_workload, operands
from test_gpu_gemm_quant_fp4 import check as check_quant

pytestmark = pytest.mark.gpu

CUS = 256


def takes_small(kind, M, N, K, batch=1):
    """The library's dispatch rule for this kernel, for one MI355X."""
    if kind == "fp4_fp4" and M <= 64:
        return False                        # the skinny MXFP4 kernel
    def tiles(bm, bn):
        return -(-M // bm) * -(-N // bn) * batch
    if 2 * tiles(256, 256) > CUS or tiles(128, 128) >= CUS or tiles(64, 64) > CUS:
        return False
    return K % 256 == 0 and 0 < K <= 1024


KIND = {("acts", "fp4"): "fp8_fp4", ("acts", "fp8"): "fp8_fp8", ("fp8", "fp4"): "fp8_fp4",
        ("fp8", "fp8"): "fp8_fp8", ("fp4", "fp4"): "fp4_fp4"}

SHAPES = [(16, 256, 512), (1024, 1024, 1024), (129, 257, 256), (65, 100, 768), (300, 520, 1024),
          (1000, 1000, 512), (1024, 1024, 256), (77, 2000, 1024)]


PAIRS = [("acts", "fp4"), ("acts", "fp8"), ("fp8", "fp4"), ("fp4", "fp4")]
# every pairing with every shape that takes this kernel for it (MXFP4 x MXFP4 with M <= 64 goes
# to the skinny kernel instead)
CASES = [(a, b, M, N, K) for (a, b) in PAIRS for (M, N, K) in SHAPES
         if takes_small(KIND[(a, b)], M, N, K)]


@pytest.mark.parametrize("a_kind,b_kind,M,N,K", CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_shapes_against_oracle(mx, a_kind, b_kind, M, N, K, with_bias):
    assert takes_small(KIND[(a_kind, b_kind)], M, N, K)
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M * 7 + N * 3 + K + with_bias,
                          with_bias=with_bias)
    check_workload(mx, w)


def test_headline_small_configurations_take_it():
    assert takes_small("fp8_fp4", 16, 256, 512)          # FP8 x MXFP4 16 x 256 x 512
    assert takes_small("fp8_fp8", 1024, 1024, 1024)      # FP8 x FP8 1024^3 + bias


@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("acts", "fp8"), ("fp4", "fp4")])
def test_batched_distinct_operands(mx, a_kind, b_kind):
    assert takes_small(KIND[(a_kind, b_kind)], 200, 300, 768, 3)
    check_workload(mx, synth.gemm_inputs(a_kind, b_kind, 200, 300, 768, seed=31, batch=3,
                                         with_bias=True))


def test_batched_shared_weight_and_bias(mx):
    # stride 0 for B, its scales and the bias
    M, N, K, nb = 130, 200, 512, 4
    assert takes_small("fp8_fp4", M, N, K, nb)
    w = synth.gemm_inputs("acts", "fp4", M, N, K, seed=32, with_bias=True)
    xs = np.stack([synth.bf16_normal(synth.rng_for(33 + i), (M, K)) for i in range(nb)])
    a = np.stack([O.act_quant(xs[i])[0] for i in range(nb)])
    a_s = np.stack([O.act_quant(xs[i])[1] for i in range(nb)])
    c = poison_bf16((nb, M, N))
    note(f"gemm fp8_fp4 batched {nb} shared weight {M}x{N}x{K}")
    mx.mx_gemm_fp8_fp4(dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s), c,
                       bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    B = O.decode_fp4_rows(w.b, w.b_s)
    bias = O.bf16_to_f64(w.bias)
    for i in range(nb):
        ref, S = O.gemm_ref(O.decode_e4m3_rows(a[i], a_s[i]), B, bias)
        assert_within(out[i], ref, S, f"batch {i}")


@pytest.mark.parametrize("epi", ["residual", "gelu"])
@pytest.mark.parametrize("a_kind,b_kind,M,N,K", [("acts", "fp8", 1024, 1024, 1024),
                                                 ("acts", "fp4", 129, 257, 256),
                                                 ("fp4", "fp4", 300, 520, 768)])
def test_epilogues(mx, epi, a_kind, b_kind, M, N, K):
    kind = KIND[(a_kind, b_kind)]
    assert takes_small(kind, M, N, K)
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M + 2 * N + K, with_bias=True)
    a, a_s, _, A, B, bias = operands(w)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    c = poison_bf16((M, N))
    note(f"gemm {kind} {epi} {M}x{N}x{K} (64x64 tiles, whole K in LDS)")
    if epi == "residual":
        res = synth.bf16_normal(synth.rng_for(M + N), (M, N))
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


@pytest.mark.parametrize("gelu", [False, True])
@pytest.mark.parametrize("a_kind,b_kind,M,N,K", [("acts", "fp4", 1024, 1024, 1024),
                                                 ("acts", "fp8", 200, 320, 512),
                                                 ("fp4", "fp4", 129, 256, 256)])
def test_quantized_outputs(mx, gelu, a_kind, b_kind, M, N, K):
    assert takes_small(KIND[(a_kind, b_kind)], M, N, K)
    check_quant(mx, synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M + N + 5 * K + gelu,
                                      with_bias=True), gelu)


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_zero_weight_gives_bias_bit_exact(mx, kind):
    M, N, K = 200, 300, 768
    assert takes_small(kind, M, N, K)
    a_k, b_k = kind.split("_")
    w = synth.gemm_inputs(a_k, b_k, M, N, K, seed=41, with_bias=True)
    c = poison_bf16((M, N))
    note(f"gemm {kind} zero weight {M}x{N}x{K}")
    getattr(mx, f"mx_gemm_{kind}")(dev_u8(w.a), dev_u8(w.a_s), dev_u8(np.zeros_like(w.b)),
                                   dev_u8(w.b_s), c, bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(c), np.broadcast_to(w.bias, (M, N)))


@pytest.mark.parametrize("M,N,K", [(129, 257, 256), (300, 520, 1024)])
def test_e5m2_e4m3_backward_operands(mx, M, N, K):
    assert takes_small("e5m2_e4m3", M, N, K)
    g = synth.bf16_normal(synth.rng_for(M + 1), (M, K), std=1e-3, outlier_frac=0.01)
    a, a_s = O.grad_quant_e5m2(g, seed=M + 1)
    wt = synth.bf16_normal(synth.rng_for(N + 2), (K, N), std=0.05)
    b, b_s = O.quant_transpose_e4m3(wt)
    c = poison_bf16((M, N))
    note(f"gemm e5m2_e4m3 {M}x{N}x{K} (64x64 tiles, whole K in LDS)")
    mx.mx_gemm_e5m2_e4m3(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), c)
    torch.cuda.synchronize()
    ref, S = O.gemm_ref(O.decode_e5m2_rows(a, a_s), O.decode_e4m3_rows(b, b_s))
    assert_within(host_bf16_bits(c), ref, S, "e5m2 x e4m3")
