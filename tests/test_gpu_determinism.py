"""Bit-determinism over 100 launches of each kind of kernel on the configurations' shapes.

Every kernel here has a fixed accumulation order per output (a tile's K steps in order, the
split-K pair added in one fp32 addition, the skinny kernel's wavefront partial sums added in
wavefront order), so 100 launches on the same inputs must give the same bytes each time.  The
outputs of every launch are compared on the device with the first launch's, bit for bit.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth

from gpu_util import dev_bf16, dev_u8, note

pytestmark = pytest.mark.gpu

REPEATS = 100


def _same_every_time(launch, outs):
    """Runs launch() REPEATS times; after each, every tensor in outs must equal its first value."""
    launch()
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    bad = []
    for i in range(1, REPEATS):
        for o in outs:
            o.fill_(0)
        launch()
        for j, (o, f) in enumerate(zip(outs, first)):
            if not torch.equal(o.view(torch.uint8), f.view(torch.uint8)):
                bad.append((i, j))
    torch.cuda.synchronize()
    assert not bad, f"launches differing from the first (launch, output): {bad[:10]}"


def _acts_operand(mx, x_bits):
    x = dev_bf16(x_bits)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=torch.uint8, device="cuda")
    mx.mx_act_quant(x, q, s)
    return x, q, s


def test_act_quant_and_gemm_4096x7168x2048(mx):
    w = synth.fp8xmxfp4_4096x7168x2048_bias()
    x, q, s = _acts_operand(mx, w.x)
    b, b_s, bias = dev_u8(w.b), dev_u8(w.b_s), dev_bf16(w.bias)
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    note("determinism: act_quant + gemm fp8_fp4 4096x7168x2048, 100 launches")

    def launch():
        mx.mx_act_quant(x, q, s)
        mx.mx_gemm_fp8_fp4(q, s, b, b_s, c, bias=bias)

    _same_every_time(launch, [q, s, c])


def test_quantized_output_gemm_4096x7168x2048(mx):
    w = synth.fp8xmxfp4_4096x7168x2048_bias()
    _, q, s = _acts_operand(mx, w.x)
    b, b_s, bias = dev_u8(w.b), dev_u8(w.b_s), dev_bf16(w.bias)
    qn = torch.empty((w.M, w.N), dtype=torch.uint8, device="cuda")
    qsn = torch.empty((w.M, w.N // 32), dtype=torch.uint8, device="cuda")
    note("determinism: gemm fp8_fp4 quant 4096x7168x2048, 100 launches")
    _same_every_time(lambda: mx.mx_gemm_fp8_fp4_quant(q, s, b, b_s, qn, qsn, bias=bias), [qn, qsn])


def test_split_k_down_projection_4096x2048x7168(mx):
    w = synth.gemm_inputs("fp8", "fp4", 4096, 2048, 7168, seed=1006, with_bias=True)
    a, a_s, b, b_s, bias = dev_u8(w.a), dev_u8(w.a_s), dev_u8(w.b), dev_u8(w.b_s), dev_bf16(w.bias)
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(mx.mx_gemm_splitk_workspace_size(w.M, w.N, w.K), dtype=torch.uint8,
                     device="cuda")
    note("determinism: gemm fp8_fp4 split-K 4096x2048x7168, 100 launches")
    _same_every_time(lambda: mx.mx_gemm_fp8_fp4_splitk(a, a_s, b, b_s, c, ws, bias=bias), [c])


def test_fp8xfp8_1024_bias_and_batched(mx):
    w1 = synth.fp8xfp8_1024cubed_bias()
    _, q1, s1 = _acts_operand(mx, w1.x)
    b1, bs1, bias1 = dev_u8(w1.b), dev_u8(w1.b_s), dev_bf16(w1.bias)
    c1 = torch.empty((w1.M, w1.N), dtype=torch.bfloat16, device="cuda")
    w2 = synth.fp8xfp8_batched_8x1024x2048x2048()
    x2 = dev_bf16(w2.x)
    q2 = torch.empty(x2.shape, dtype=torch.uint8, device="cuda")
    s2 = torch.empty(x2.shape[:-1] + (x2.shape[-1] // 32,), dtype=torch.uint8, device="cuda")
    mx.mx_act_quant_strided_batched(x2, q2, s2)
    b2, bs2 = dev_u8(w2.b), dev_u8(w2.b_s)
    c2 = torch.empty((w2.batch, w2.M, w2.N), dtype=torch.bfloat16, device="cuda")
    note("determinism: gemm fp8_fp8 1024^3 + bias and batched 8x1024x2048x2048, 100 launches")

    def launch():
        mx.mx_gemm_fp8_fp8(q1, s1, b1, bs1, c1, bias=bias1)
        mx.mx_gemm_fp8_fp8(q2, s2, b2, bs2, c2)

    _same_every_time(launch, [c1, c2])


@pytest.mark.parametrize("i", [0, 1, 2])
def test_skinny_a4w4(mx, i):
    w = synth.a4w4_skinny(i)
    a, a_s, b, b_s = dev_u8(w.a), dev_u8(w.a_s), dev_u8(w.b), dev_u8(w.b_s)
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    note(f"determinism: gemm fp4_fp4 {w.M}x{w.N}x{w.K}, 100 launches")
    _same_every_time(lambda: mx.mx_gemm_fp4_fp4(a, a_s, b, b_s, c), [c])


def test_outputs_are_not_trivially_constant(mx):
    # The comparisons above would pass on an all-zero output; the C5 GEMM's output is not one.
    w = synth.fp8xmxfp4_4096x7168x2048_bias()
    _, q, s = _acts_operand(mx, w.x)
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    mx.mx_gemm_fp8_fp4(q, s, dev_u8(w.b), dev_u8(w.b_s), c, bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    vals = c.float().cpu().numpy()
    assert np.isfinite(vals).all() and np.unique(vals[:64, :64]).size > 1000
