"""GEMM residual and GELU epilogues on the GPU against the oracle (O6).

Residual outputs must meet the GEMM bound |out - ref| <= 2^-7 |ref| + 2^-20 S against the exact
ref = sum a*b + bias + residual; GELU outputs must meet |out - gelu(pre)| <= 2^-7 |gelu(pre)| +
2^-19 S + 2^-126 against the exact pre = sum a*b + bias.  Operands quantized from activations are
quantized by the oracle, so no oracle input comes from the GPU.  With zero weights the residual
output is a closed form and must match bit for bit.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16

pytestmark = pytest.mark.gpu

KIND = {("fp8", "fp4"): "fp8_fp4", ("fp8", "fp8"): "fp8_fp8", ("fp4", "fp4"): "fp4_fp4"}


def operands(w: synth.GemmWorkload):
    lead = w.batch is not None
    if w.a_kind == "acts":
        a, a_s = O.act_quant(w.x)
        a_kind = "fp8"
    else:
        a, a_s, a_kind = w.a, w.a_s, w.a_kind
    dec_a = O.decode_fp4_rows if a_kind == "fp4" else O.decode_e4m3_rows
    dec_b = O.decode_fp4_rows if w.b_kind == "fp4" else O.decode_fp8_block
    if lead:
        A = np.stack([dec_a(a[i], a_s[i]) for i in range(w.batch)])
        B = np.stack([dec_b(w.b[i], w.b_s[i]) for i in range(w.batch)])
    else:
        A, B = dec_a(a, a_s), dec_b(w.b, w.b_s)
    bias = None if w.bias is None else O.bf16_to_f64(w.bias)
    return a, a_s, KIND[(a_kind, w.b_kind)], A, B, bias


def run(mx, kind, epi, a, a_s, b, b_s, bias, residual, shape, in_place=False):
    if in_place:
        c = dev_bf16(residual)
        res = c
    else:
        c = poison_bf16(shape)
        res = None if residual is None else dev_bf16(residual)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s))
    bias_t = None if bias is None else dev_bf16(bias)
    if epi == "residual":
        getattr(mx, f"mx_gemm_{kind}_bias_residual")(*args, res, c, bias=bias_t)
    else:
        getattr(mx, f"mx_gemm_{kind}_bias_gelu")(*args, c, bias=bias_t)
    torch.cuda.synchronize()
    return host_bf16_bits(c)


def check(out, epi, A, B, bias, residual, what):
    if epi == "residual":
        ref, S = O.gemm_residual_ref(A, B, bias, residual)
        ok = O.within_tolerance(out, ref, S)
        pre = ref
    else:
        _, pre, S = O.gemm_gelu_ref(A, B, bias)
        ok = O.gelu_within(out, pre, S)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        got = O.bf16_to_f64(out)
        pytest.fail(f"{what}: {np.count_nonzero(~ok)} of {ok.size} outside the bound; first "
                    f"(index, gpu, pre, S): {[(tuple(i), got[tuple(i)], pre[tuple(i)], S[tuple(i)]) for i in idx]}")


SHAPES = [(1, 1, 32), (1, 31, 64), (41, 33, 96), (64, 64, 64), (129, 257, 160), (100, 300, 1024),
          (33, 65, 2080), (300, 520, 256)]


@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("acts", "fp8"), ("fp4", "fp4")])
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("epi", ["residual", "gelu"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_ragged_shapes(mx, a_kind, b_kind, M, N, K, epi, with_bias):
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M * 131 + N * 17 + K + with_bias,
                          with_bias=with_bias, bias_std=1.0)
    a, a_s, kind, A, B, bias = operands(w)
    residual = synth.bf16_normal(synth.rng_for(M + N + K), (M, N)) if epi == "residual" else None
    note(f"gemm {kind} {epi} M={M} N={N} K={K} bias={with_bias}")
    out = run(mx, kind, epi, a, a_s, w.b, w.b_s, w.bias, residual, (M, N))
    check(out, epi, A, B, bias, residual, f"{kind} {epi} {M}x{N}x{K}")


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
@pytest.mark.parametrize("M,N,K", [(41, 4608, 1536), (257, 515, 192)])
def test_residual_in_place(mx, kind, M, N, K):
    # c is the residual: out = sum + bias + c, written over c.
    a_k, b_k = kind.split("_")
    w = synth.gemm_inputs(a_k, b_k, M, N, K, seed=77 + M, with_bias=True)
    a, a_s, kind, A, B, bias = operands(w)
    residual = synth.bf16_normal(synth.rng_for(78 + M), (M, N))
    note(f"gemm {kind} residual in place {M}x{N}x{K}")
    out = run(mx, kind, "residual", a, a_s, w.b, w.b_s, w.bias, residual, (M, N), in_place=True)
    check(out, "residual", A, B, bias, residual, "in place")


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_zero_weight_residual_bit_exact(mx, kind):
    # sum = 0, so out = bf16_rne(bias + residual): one rounding of a sum that is exact in fp32.
    M, N, K = 70, 200, 96
    a_k, b_k = kind.split("_")
    w = synth.gemm_inputs(a_k, b_k, M, N, K, seed=13, with_bias=True, bias_std=1.0)
    residual = synth.bf16_normal(synth.rng_for(14), (M, N))
    exact = O.bf16_to_f64(w.bias)[None, :] + O.bf16_to_f64(residual)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    note(f"gemm zero weight residual {kind}")
    out = run(mx, kind, "residual", w.a, w.a_s, np.zeros_like(w.b), w.b_s, w.bias, residual,
              (M, N))
    assert np.array_equal(out, O.f64_to_bf16_rne(exact))


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_zero_weight_gelu_of_bias(mx, kind):
    # sum = 0, so out = bf16(gelu(bias)) within 2^-7 relative (S = 0); bias spans [-12, 12].
    M, N, K = 40, 1024, 64
    a_k, b_k = kind.split("_")
    w = synth.gemm_inputs(a_k, b_k, M, N, K, seed=15, with_bias=True)
    bias = (np.linspace(-12, 12, N).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    note(f"gemm zero weight gelu {kind}")
    out = run(mx, kind, "gelu", w.a, w.a_s, np.zeros_like(w.b), w.b_s, bias, None, (M, N))
    pre = np.broadcast_to(O.bf16_to_f64(bias), (M, N))
    assert O.gelu_within(out, pre, np.zeros((M, N))).all()
    assert np.all(O.bf16_to_f64(out[:, -1]) == O.bf16_to_f64(bias[-1]))   # gelu(12) = 12 in bf16


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp4_fp4"])
def test_gelu_of_every_bf16_value_in_range(mx, kind):
    # Zero weights make the pre-activation exactly the bias: every finite bf16 value with
    # |x| <= 16 (both signs, subnormals included) goes through the kernel's GELU once.
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(b)
    bias = b[np.isfinite(v) & (np.abs(v) <= 16)]
    N, M, K = len(bias), 3, 64
    a_k, b_k = kind.split("_")
    w = synth.gemm_inputs(a_k, b_k, M, N, K, seed=16)
    note(f"gemm gelu every bf16 in [-16, 16] {kind} N={N}")
    out = run(mx, kind, "gelu", w.a, w.a_s, np.zeros_like(w.b), w.b_s, bias, None, (M, N))
    pre = np.broadcast_to(O.bf16_to_f64(bias), (M, N))
    ok = O.gelu_within(out, pre, np.zeros((M, N)))
    assert ok.all(), [(hex(bias[j]), hex(out[0, j])) for j in np.nonzero(~ok[0])[0][:8]]


@pytest.mark.parametrize("epi", ["residual", "gelu"])
@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("fp4", "fp4")])
def test_batched_with_broadcast_residual_and_bias(mx, epi, a_kind, b_kind):
    B_, M, N, K = 3, 70, 96, 192
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=44, batch=B_, with_bias=True)
    a, a_s, kind, A, B, bias = operands(w)
    c = poison_bf16((B_, M, N))
    res2 = synth.bf16_normal(synth.rng_for(45), (M, N))
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    note(f"gemm {kind} {epi} batched")
    if epi == "residual":
        res = dev_bf16(res2).unsqueeze(0).expand(B_, M, N)          # stride 0 over the batch
        getattr(mx, f"mx_gemm_{kind}_bias_residual")(*args, res, c, bias=dev_bf16(w.bias))
    else:
        getattr(mx, f"mx_gemm_{kind}_bias_gelu")(*args, c, bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    for i in range(B_):
        check(out[i], epi, A[i], B[i], bias[i], res2 if epi == "residual" else None, f"batch {i}")


@pytest.mark.parametrize("epi", ["residual", "gelu"])
def test_fp8xmxfp4_4096x7168x2048_sampled(mx, epi):
    w = synth.fp8xmxfp4_4096x7168x2048_bias()
    a, a_s = O.act_quant(w.x)
    residual = synth.bf16_normal(synth.rng_for(2024), (w.M, w.N)) if epi == "residual" else None
    note(f"gemm fp8_fp4 {epi} 4096x7168x2048")
    out = run(mx, "fp8_fp4", epi, a, a_s, w.b, w.b_s, w.bias, residual, (w.M, w.N))
    assert np.isfinite(O.bf16_to_f64(out)).all()
    rows = np.random.default_rng(5).integers(0, w.M, 3000)
    cols = np.random.default_rng(6).integers(0, w.N, 3000)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    A = O.decode_e4m3_rows(a[ur], a_s[ur])
    B = O.decode_fp4_rows(w.b[uc], w.b_s[uc])
    pre, S = O.gemm_ref_at(A, B, ri, ci, O.bf16_to_f64(w.bias)[uc])
    if epi == "residual":
        ref = pre + O.bf16_to_f64(residual[rows, cols])
        assert O.within_tolerance(out[rows, cols], ref, S).all()
    else:
        assert O.gelu_within(out[rows, cols], pre, S).all()


def test_plain_entry_points_unchanged_by_epilogue_calls(mx):
    # Interleaving epilogue calls with the plain bias entry point leaves its output bit-identical.
    w = synth.gemm_inputs("acts", "fp8", 300, 200, 512, seed=5, with_bias=True)
    a, a_s, kind, A, B, bias = operands(w)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    outs = []
    for _ in range(3):
        c = poison_bf16((300, 200))
        mx.mx_gemm_fp8_fp8(*args, c, bias=dev_bf16(w.bias))
        g = poison_bf16((300, 200))
        mx.mx_gemm_fp8_fp8_bias_gelu(*args, g, bias=dev_bf16(w.bias))
        torch.cuda.synchronize()
        outs.append(host_bf16_bits(c))
    assert all(np.array_equal(o, outs[0]) for o in outs)
