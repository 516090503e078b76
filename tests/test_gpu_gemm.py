"""Block-scaled GEMMs on the GPU against the oracle.

Every GPU output must satisfy |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k| against the exact
float64 reference computed from the same bytes; the closed forms (identity and zero weights)
must match bit for bit.  A operands that come from activations are quantized by the ORACLE here,
so no oracle input ever comes from the GPU; the pipeline test quantizes on the GPU and is
checked against the oracle's own pipeline.
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
    """(a_bytes, a_scales, A f64, B f64, bias f64|None) from the workload's bytes, via the oracle."""
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
    return a, a_s, a_kind, A, B, bias


def run(mx, kind, a, a_s, b, b_s, bias, M, N, batch=None):
    fn = getattr(mx, f"mx_gemm_{kind}")
    shape = (M, N) if batch is None else (batch, M, N)
    c = poison_bf16(shape)
    fn(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), c,
       bias=None if bias is None else dev_bf16(bias))
    torch.cuda.synchronize()
    return host_bf16_bits(c)


def assert_within(out_bits, ref, S, what=""):
    ok = O.within_tolerance(out_bits, ref, S)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        out = O.bf16_to_f64(out_bits)
        detail = [(tuple(i), out[tuple(i)], ref[tuple(i)], S[tuple(i)]) for i in idx]
        pytest.fail(f"{what}: {np.count_nonzero(~ok)} of {ok.size} outputs outside the bound; "
                    f"first (index, gpu, ref, S): {detail}")


def check_workload(mx, w: synth.GemmWorkload):
    a, a_s, a_kind, A, B, bias = operands(w)
    kind = KIND[(a_kind, w.b_kind)]
    note(f"gemm {kind} {w.name} batch={w.batch}")
    out = run(mx, kind, a, a_s, w.b, w.b_s, w.bias, w.M, w.N, w.batch)
    ref, S = O.gemm_ref(A, B, bias)
    assert_within(out, ref, S, w.name)


SHAPES = [(1, 1, 32), (1, 31, 64), (41, 33, 96), (64, 64, 64), (129, 257, 160), (100, 300, 1024),
          (33, 65, 2080)]


@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("acts", "fp8"), ("fp8", "fp8"),
                                           ("fp8", "fp4"), ("fp4", "fp4")])
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_ragged_shapes(mx, a_kind, b_kind, M, N, K, with_bias):
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M * 7919 + N * 31 + K + with_bias,
                          with_bias=with_bias)
    check_workload(mx, w)


@pytest.mark.parametrize("a_kind,b_kind", [("acts", "fp4"), ("acts", "fp8"), ("fp4", "fp4")])
@pytest.mark.parametrize("with_bias", [False, True])
def test_batched_distinct_operands(mx, a_kind, b_kind, with_bias):
    w = synth.gemm_inputs(a_kind, b_kind, 70, 96, 192, seed=42, batch=3, with_bias=with_bias)
    check_workload(mx, w)


@pytest.mark.parametrize("b_kind", ["fp4", "fp8"])
def test_batched_broadcast_weight_and_bias(mx, b_kind):
    # The weight, its scales and the bias are shared by every batch (stride 0).
    B_, M, N, K = 4, 50, 70, 128
    w = synth.gemm_inputs("acts", b_kind, M, N, K, seed=8, batch=B_, with_bias=True)
    a, a_s = O.act_quant(w.x)
    b0, bs0, bias0 = w.b[0], w.b_s[0], w.bias[0]
    kind = KIND[("fp8", b_kind)]
    c = poison_bf16((B_, M, N))
    note(f"gemm {kind} broadcast weight")
    getattr(mx, f"mx_gemm_{kind}")(dev_u8(a), dev_u8(a_s), dev_u8(b0), dev_u8(bs0), c,
                                   bias=dev_bf16(bias0))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    Bd = O.decode_fp4_rows(b0, bs0) if b_kind == "fp4" else O.decode_fp8_block(b0, bs0)
    for i in range(B_):
        ref, S = O.gemm_ref(O.decode_e4m3_rows(a[i], a_s[i]), Bd, O.bf16_to_f64(bias0))
        assert_within(out[i], ref, S, f"batch {i}")


@pytest.mark.parametrize("b_kind", ["fp4", "fp8"])
def test_identity_weight_gives_act_qdq_bit_exact(mx, b_kind):
    # B = I (scale 1.0): every output is one exact product, the act_qdq value, a bf16 value.
    M, K = 100, 256
    x = synth.bf16_normal(synth.rng_for(31), (M, K), outlier_frac=0.05)
    a, a_s = O.act_quant(x)
    if b_kind == "fp8":
        b = np.zeros((K, K), np.uint8)
        np.fill_diagonal(b, 0x38)
        b_s = np.full((K // 32, K // 32), 127, np.uint8)
        kind = "fp8_fp8"
    else:
        cds = np.zeros((K, K), np.uint8)
        np.fill_diagonal(cds, 2)
        b = (cds[:, 0::2] | (cds[:, 1::2] << 4)).astype(np.uint8)
        b_s = np.full((K, K // 32), 127, np.uint8)
        kind = "fp8_fp4"
    note(f"gemm identity {kind}")
    out = run(mx, kind, a, a_s, b, b_s, None, M, K)
    qdq = O.act_qdq_f64(a, a_s)
    # Bit-exact values; a -0 activation comes back as +0 (+0 accumulator plus -0 product).
    want = (qdq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    zero = qdq == 0
    assert np.array_equal(out[~zero], want[~zero])
    assert np.all(O.bf16_to_f64(out[zero]) == 0)


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8", "fp4_fp4"])
def test_zero_weight_gives_bias_bit_exact(mx, kind):
    M, N, K = 65, 130, 96
    rng = synth.rng_for(12)
    a_k, b_k = kind.split("_")
    w = synth.gemm_inputs(a_k, b_k, M, N, K, seed=12, with_bias=True)
    b = np.zeros_like(w.b)
    note(f"gemm zero weight {kind}")
    out = run(mx, kind, w.a, w.a_s, b, w.b_s, w.bias, M, N)
    assert np.array_equal(out, np.broadcast_to(w.bias, (M, N)))


# Wide outputs of 448 tiles of 256x256 with ragged M, N and K edges (1.75 waves on 256 CUs).
WIDE_CASES = [("acts", "fp4", 500, 57267, 224, None, True),
               ("acts", "fp8", 256, 57344, 256, 2, False),
               ("fp8", "fp4", 511, 57300, 96, None, True),
               ("fp4", "fp4", 300, 57344, 128, None, True)]


@pytest.mark.parametrize("a_kind,b_kind,M,N,K,batch,with_bias", WIDE_CASES)
def test_wide_ragged_shapes(mx, a_kind, b_kind, M, N, K, batch, with_bias):
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M + N + K, batch=batch,
                          with_bias=with_bias)
    check_workload(mx, w)


def test_headline_fp8xmxfp4_16x256x512(mx):
    check_workload(mx, synth.fp8xmxfp4_16x256x512())


def test_headline_fp8xfp8_1024_bias(mx):
    check_workload(mx, synth.fp8xfp8_1024cubed_bias())


@pytest.mark.parametrize("i", [0, 1, 2])
def test_headline_skinny_a4w4(mx, i):
    check_workload(mx, synth.a4w4_skinny(i))


def test_headline_batched_8x1024x2048x2048(mx):
    check_workload(mx, synth.fp8xfp8_batched_8x1024x2048x2048())


def test_headline_fp8xmxfp4_4096x7168x2048_bias(mx):
    check_workload(mx, synth.fp8xmxfp4_4096x7168x2048_bias())


def test_headline_fp8xfp8_8192_full(mx):
    # The longest accumulation of the configurations (K = 8192): every one of the 67,108,864
    # outputs against the float64 reference.
    check_workload(mx, synth.fp8xfp8_8192cubed())


def test_pipeline_act_quant_then_gemm_4096x7168x2048(mx):
    # act_quant and the GEMM back to back on one stream, on the GPU, against the oracle's
    # own pipeline (oracle act_quant, then the float64 GEMM).
    w = synth.fp8xmxfp4_4096x7168x2048_bias()
    x = dev_bf16(w.x)
    q = torch.empty((w.M, w.K), dtype=torch.uint8, device="cuda")
    s = torch.empty((w.M, w.K // 32), dtype=torch.uint8, device="cuda")
    c = poison_bf16((w.M, w.N))
    note("pipeline act_quant -> gemm fp8_fp4 4096x7168x2048")
    mx.mx_act_quant(x, q, s)
    mx.mx_gemm_fp8_fp4(q, s, dev_u8(w.b), dev_u8(w.b_s), c, bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    a, a_s = O.act_quant(w.x)
    ref, S = O.gemm_ref(O.decode_e4m3_rows(a, a_s), O.decode_fp4_rows(w.b, w.b_s),
                        O.bf16_to_f64(w.bias))
    assert_within(out, ref, S, "pipeline")


def test_repeat_deterministic(mx):
    w = synth.gemm_inputs("acts", "fp8", 300, 200, 512, seed=5, with_bias=True)
    a, a_s, _, _, _, _ = operands(w)
    outs = [run(mx, "fp8_fp8", a, a_s, w.b, w.b_s, w.bias, w.M, w.N) for _ in range(5)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("kind,a_kind,b_kind", [("fp8_fp4", "acts", "fp4"), ("fp8_fp8", "acts", "fp8"),
                                                ("fp4_fp4", "fp4", "fp4")])
def test_output_with_unaligned_base_matches_aligned(mx, kind, a_kind, b_kind):
    # C needs no alignment: an output starting 2 bytes past a 16-byte boundary takes the
    # copy-out's per-chunk path and must hold exactly the bytes the aligned output gets from the
    # 16-byte-store path (same kernel, same sums).  M = 512 > 64 runs the tiled kernel for every
    # kind, with whole 256x256 tiles.
    M, N, K = 512, 512, 256
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=77, with_bias=True)
    a, a_s, _, A, B, bias = operands(w)
    note(f"gemm {kind} unaligned output base")
    aligned = run(mx, kind, a, a_s, w.b, w.b_s, w.bias, M, N)
    big = torch.full((M * N + 8,), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    c = big[1:1 + M * N].view(M, N)
    assert c.data_ptr() % 16 == 2
    getattr(mx, f"mx_gemm_{kind}")(dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s), c,
                                   bias=dev_bf16(w.bias))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(c), aligned)
    assert int(big[0].view(torch.int16)) == -1 and int(big[-1].view(torch.int16)) == -1
    assert_within(aligned, *O.gemm_ref(A, B, bias))
