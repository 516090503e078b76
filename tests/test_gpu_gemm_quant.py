"""GEMMs whose output is the next layer's activation operand (E4M3 codes + per-32 E8M0 bytes).

Two checks per case:
* bit-exact against the composition of two separately tested GPU paths: the bf16 GEMM followed by
  act_quant on its output (the quantizing epilogue must reproduce exactly those bytes);
* against the oracle: every dequantized output is within the bound quant_output_within derives
  from the GEMM tolerance and the E4M3 rounding, and every scale byte is within one of the scale
  act_quant gives the oracle's own bf16 rounding of the exact result.
A operands that come from activations are quantized by the oracle, as in the bf16 GEMM tests.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16
from test_gpu_gemm import operands

pytestmark = pytest.mark.gpu


def _poison_u8(shape):
    return torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")     # an E4M3 NaN code


def run_quant(mx, kind, a, a_s, b, b_s, bias, M, N, batch=None):
    shape = (M, N) if batch is None else (batch, M, N)
    q = _poison_u8(shape)
    qs = torch.full(shape[:-1] + (N // 32,), 0xFF, dtype=torch.uint8, device="cuda")
    getattr(mx, f"mx_gemm_{kind}_quant")(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), q, qs,
                                         bias=None if bias is None else dev_bf16(bias))
    torch.cuda.synchronize()
    return q.cpu().numpy(), qs.cpu().numpy()


def run_unfused(mx, kind, a, a_s, b, b_s, bias, M, N, batch=None):
    shape = (M, N) if batch is None else (batch, M, N)
    c = poison_bf16(shape)
    getattr(mx, f"mx_gemm_{kind}")(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), c,
                                   bias=None if bias is None else dev_bf16(bias))
    q = torch.empty(shape, dtype=torch.uint8, device="cuda")
    qs = torch.empty(shape[:-1] + (N // 32,), dtype=torch.uint8, device="cuda")
    if batch is None:
        mx.mx_act_quant(c, q, qs)
    else:
        mx.mx_act_quant_strided_batched(c, q, qs)
    torch.cuda.synchronize()
    return q.cpu().numpy(), qs.cpu().numpy(), host_bf16_bits(c)


def check(mx, w):
    a, a_s, a_kind, A, B, bias = operands(w)
    kind = f"{a_kind}_{w.b_kind}"
    note(f"gemm quant {kind} {w.name} batch={w.batch}")
    q, qs = run_quant(mx, kind, a, a_s, w.b, w.b_s, w.bias, w.M, w.N, w.batch)
    q2, qs2, _ = run_unfused(mx, kind, a, a_s, w.b, w.b_s, w.bias, w.M, w.N, w.batch)
    assert np.array_equal(q, q2), f"{w.name}: codes differ from gemm + act_quant"
    assert np.array_equal(qs, qs2), f"{w.name}: scale bytes differ from gemm + act_quant"
    ref, S, _, _, oscales = O.gemm_act_quant_ref(A, B, bias)
    ok = O.quant_output_within(q, qs, ref, S)
    assert ok.all(), f"{w.name}: {np.count_nonzero(~ok)} of {ok.size} outputs outside the bound"
    assert np.abs(qs.astype(int) - oscales.astype(int)).max() <= 1


SHAPES = [(1, 32, 32), (41, 96, 96), (129, 256, 160), (300, 544, 1024), (33, 64, 2080),
          (257, 320, 224)]


@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("acts", "fp8"), ("fp8", "fp4")])
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_quant_output_shapes(mx, a_kind, b_kind, M, N, K, with_bias):
    check(mx, synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M * 31 + N + K + 7 * with_bias,
                                with_bias=with_bias))


@pytest.mark.parametrize("b_kind", ["fp4", "fp8"])
def test_quant_output_batched(mx, b_kind):
    check(mx, synth.gemm_inputs("acts", b_kind, 70, 96, 192, seed=43, batch=3, with_bias=True))


def test_quant_output_rejects_ragged_n(mx):
    w = synth.gemm_inputs("fp8", "fp4", 16, 48, 64, seed=3)
    q = torch.empty((16, 48), dtype=torch.uint8, device="cuda")
    qs = torch.empty((16, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError) as e:
        mx.mx_gemm_fp8_fp4_quant(dev_u8(w.a), dev_u8(w.a_s), dev_u8(w.b), dev_u8(w.b_s), q, qs)
    assert e.value.status == mx.MX_ERR_SHAPE


def test_quant_output_fp8xmxfp4_4096x7168x2048_bias(mx):
    check(mx, synth.fp8xmxfp4_4096x7168x2048_bias())


def test_quant_output_fp8xfp8_1024_bias(mx):
    check(mx, synth.fp8xfp8_1024cubed_bias())
