"""GEMMs whose output is the next layer's operand, quantized in the epilogue: MXFP4 (packed E2M1 +
per-32 E8M0) from the A4W4 GEMM, and bias + GELU followed by the quantization of every kind
(MXFP4 for the A4W4 GEMM, the E4M3 activation operand for the FP8 ones).

Two checks per case, as for the E4M3 quantizing epilogue:
* bit-exact against the composition of two separately tested GPU paths: the bf16 GEMM (with the
  GELU epilogue where asked) followed by the matching activation quantizer on its output;
* against the oracle: every dequantized output is within the bound that the MXFP4 (or E4M3)
  rounding adds to the bf16 bound (the GEMM bound, or the GELU bound after GELU), and every scale
  byte is within one of the scale the oracle's own bf16 rounding of the exact result gives.
The MXFP4 GEMM takes the skinny kernel for M <= 64 (both of its wavefront counts: K below and from
4096 on) and the tiled kernel above.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16
from test_gpu_gemm import operands

pytestmark = pytest.mark.gpu


def _out_cols(kind, N):
    return N // 2 if kind == "fp4_fp4" else N


def run_fused(mx, kind, gelu, a, a_s, b, b_s, bias, M, N, batch=None):
    lead = () if batch is None else (batch,)
    q = torch.full(lead + (M, _out_cols(kind, N)), 0x7F, dtype=torch.uint8, device="cuda")
    qs = torch.full(lead + (M, N // 32), 0xFF, dtype=torch.uint8, device="cuda")
    name = f"mx_gemm_{kind}_bias_gelu_quant" if gelu else f"mx_gemm_{kind}_quant"
    getattr(mx, name)(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), q, qs,
                      bias=None if bias is None else dev_bf16(bias))
    torch.cuda.synchronize()
    return q.cpu().numpy(), qs.cpu().numpy()


def run_unfused(mx, kind, gelu, a, a_s, b, b_s, bias, M, N, batch=None):
    lead = () if batch is None else (batch,)
    c = poison_bf16(lead + (M, N))
    name = f"mx_gemm_{kind}_bias_gelu" if gelu else f"mx_gemm_{kind}"
    getattr(mx, name)(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), c,
                      bias=None if bias is None else dev_bf16(bias))
    q = torch.empty(lead + (M, _out_cols(kind, N)), dtype=torch.uint8, device="cuda")
    qs = torch.empty(lead + (M, N // 32), dtype=torch.uint8, device="cuda")
    quant = "mx_act_quant_fp4" if kind == "fp4_fp4" else "mx_act_quant"
    if batch is not None:
        quant += "_strided_batched"
    getattr(mx, quant)(c, q, qs)
    torch.cuda.synchronize()
    return q.cpu().numpy(), qs.cpu().numpy()


def _oracle_check(kind, gelu, q, qs, A, B, bias, what):
    if kind == "fp4_fp4":
        ref, S, _, _, oscales = O.gemm_quant_fp4_ref(A, B, bias, gelu=gelu)
        if gelu:
            t = O.gelu_output_bound(ref, S)
        else:
            t = np.ldexp(np.abs(ref), -7) + np.ldexp(S, -20)
        ok = O.quant_fp4_output_within(q, qs, ref, t)
    else:
        pre, S = O.gemm_ref(A, B, bias)
        ref = O.gelu_f64(pre) if gelu else pre
        oscales = O.act_quant(O.f64_to_bf16_rne(ref))[1]
        ok = O.quant_output_within(q, qs, ref, S, t=O.gelu_output_bound(ref, S) if gelu else None)
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} of {ok.size} outputs outside the bound"
    assert np.abs(qs.astype(int) - oscales.astype(int)).max() <= 1, what


def check(mx, w, gelu):
    a, a_s, a_kind, A, B, bias = operands(w)
    kind = f"{a_kind}_{w.b_kind}"
    what = f"{kind} gelu={gelu} {w.name} batch={w.batch}"
    note(f"gemm quant-out {what}")
    q, qs = run_fused(mx, kind, gelu, a, a_s, w.b, w.b_s, w.bias, w.M, w.N, w.batch)
    q2, qs2 = run_unfused(mx, kind, gelu, a, a_s, w.b, w.b_s, w.bias, w.M, w.N, w.batch)
    assert np.array_equal(q, q2), f"{what}: codes differ from the unfused pair"
    assert np.array_equal(qs, qs2), f"{what}: scale bytes differ from the unfused pair"
    if w.batch is None:
        _oracle_check(kind, gelu, q, qs, A, B, bias, what)
    else:
        for i in range(w.batch):
            _oracle_check(kind, gelu, q[i], qs[i], A[i], B[i],
                          None if bias is None else bias[i], f"{what}[{i}]")


# Skinny (M <= 64): one to four 16-row tiles, K under and over the 8-wavefront threshold
# (4096); tiled: M from 65 on, with row and column tails.
FP4_SHAPES = [(1, 32, 64), (16, 4608, 1536), (41, 96, 6144), (64, 320, 4096), (33, 64, 2080),
              (65, 64, 128), (129, 256, 160), (300, 544, 1024)]


@pytest.mark.parametrize("M,N,K", FP4_SHAPES)
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("gelu", [False, True])
def test_fp4_output_shapes(mx, M, N, K, with_bias, gelu):
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=M * 13 + N + K + 5 * with_bias + gelu,
                          with_bias=with_bias)
    check(mx, w, gelu)


@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("acts", "fp8")])
@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (41, 96, 96), (129, 256, 160), (300, 544, 1024)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_gelu_quant_fp8_kinds(mx, a_kind, b_kind, M, N, K, with_bias):
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M * 7 + N + K + with_bias,
                          with_bias=with_bias)
    check(mx, w, gelu=True)


@pytest.mark.parametrize("M", [24, 200])
@pytest.mark.parametrize("gelu", [False, True])
def test_fp4_output_batched(mx, M, gelu):
    check(mx, synth.gemm_inputs("fp4", "fp4", M, 96, 256, seed=M + gelu, batch=3, with_bias=True),
          gelu)


def test_gelu_quant_fp8_batched(mx):
    check(mx, synth.gemm_inputs("acts", "fp4", 70, 96, 192, seed=47, batch=3, with_bias=True),
          gelu=True)


def test_fp4_output_a4w4_decode_shape(mx):
    # a decode-like A4W4 up-projection: 32 tokens x 4608 outputs x 7168 inputs, bias + GELU
    check(mx, synth.gemm_inputs("fp4", "fp4", 32, 4608, 7168, seed=9, with_bias=True), gelu=True)


@pytest.mark.parametrize("M", [8, 100])
def test_fp4_output_rejects_ragged_n(mx, M):
    w = synth.gemm_inputs("fp4", "fp4", M, 48, 64, seed=3)
    q = torch.empty((M, 24), dtype=torch.uint8, device="cuda")
    qs = torch.empty((M, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError) as e:
        mx.mx_gemm_fp4_fp4_quant(dev_u8(w.a), dev_u8(w.a_s), dev_u8(w.b), dev_u8(w.b_s), q, qs)
    assert e.value.status == mx.MX_ERR_SHAPE


# The large-problem kernel (256 x 256 or 256 x 224 tiles) quantizes straight from its
# accumulators: MXFP4 output from an FP4 A operand, and the E4M3 output after GELU.
@pytest.mark.parametrize("a_kind,M,N,K", [("fp4", 2048, 7168, 512), ("fp4", 4096, 4096, 1024),
                                          ("acts", 2048, 7168, 512), ("acts", 4000, 4096, 512)])
@pytest.mark.parametrize("gelu", [False, True])
def test_large_kernel_quantized_outputs(mx, a_kind, M, N, K, gelu):
    w = synth.gemm_inputs(a_kind, "fp4", M, N, K, seed=M + N + K + gelu, with_bias=True)
    check(mx, w, gelu)
