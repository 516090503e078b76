"""Backward-pass operands and GEMM on the GPU against the oracle (O7).

The E5M2 quantizer (round-to-nearest-even and stochastic) and both quantize-transposes must match
the oracle byte for byte, codes and scale bytes: the stochastic draws come from the same
Philox4x64-10 stream on both sides.  The E5M2 x E4M3 GEMM must meet the GEMM bound against the
exact product of the decoded operands, and the dX / dW pipeline of a linear layer is checked end
to end against the oracle's own pipeline.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, host_u8, note, poison_bf16

pytestmark = pytest.mark.gpu


def run_quant(mx, x_bits, seed=None):
    shape = x_bits.shape
    x = dev_bf16(x_bits)
    q = torch.full(shape, 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full(shape[:-1] + (shape[-1] // 32,), 0xAA, dtype=torch.uint8, device="cuda")
    mx.mx_quant_e5m2(x, q, s, seed=seed)
    torch.cuda.synchronize()
    return host_u8(q), host_u8(s)


def run_transpose(mx, x_bits, fmt, seed=None):
    R, C = x_bits.shape
    x = dev_bf16(x_bits)
    q = torch.full((C, R), 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full((C, R // 32), 0xAA, dtype=torch.uint8, device="cuda")
    if fmt == "e4m3":
        mx.mx_quant_transpose_e4m3(x, q, s)
    else:
        mx.mx_quant_transpose_e5m2(x, q, s, seed=seed)
    torch.cuda.synchronize()
    return host_u8(q), host_u8(s)


def assert_bytes(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} bytes differ, first {[(tuple(i), int(got[tuple(i)]), int(want[tuple(i)])) for i in bad[:6]]}"


def _finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def _exhaustive_blocks(step=1):
    """Every finite bf16 value under every scale exponent E in [-127, 113] (every `step`-th, and
    113): each block's first element is 57344 * 2^E (the largest bf16 for E = 113, where that
    overflows), the other 31 run through every finite bf16 with |x| <= that, so the block's scale
    is exactly 2^E; plus blocks of bf16 subnormals and zeros, whose scale is clamped to 2^-127."""
    b = _finite_bf16()
    mag = O.bf16_to_f64(b & 0x7FFF)
    blocks = []
    for E in list(range(-127, 113, step)) + [113]:
        lim = 57344.0 * 2.0 ** E
        if lim > float(np.finfo(np.float32).max):          # E = 113: the top binade of bf16
            head, lim = np.array([0x7F7F], np.uint16), np.inf
        else:
            head = (np.array([lim], np.float32).view(np.uint32) >> 16).astype(np.uint16)
        vals = b[mag <= lim]
        n = -(-len(vals) // 31)
        body = np.zeros(n * 31, np.uint16)
        body[:len(vals)] = vals
        blocks.append(np.concatenate([np.repeat(head, n)[:, None], body.reshape(n, 31)], axis=1))
    sub = b[(b & 0x7F80) == 0]                              # zeros and subnormals, both signs
    sub = np.concatenate([sub, np.zeros((-len(sub)) % 32, np.uint16)])
    blocks.append(sub.reshape(-1, 32))
    allb = np.concatenate(blocks, axis=0)
    allb = np.concatenate([allb, np.zeros(((-len(allb)) % 32, 32), np.uint16)], axis=0)
    return allb.reshape(-1, 1024)


def test_e5m2_rne_exhaustive_bf16_times_scales(mx):
    x = _exhaustive_blocks()
    note(f"quant_e5m2 rne exhaustive {x.shape}")
    q, s = run_quant(mx, x)
    rq, rs = O.grad_quant_e5m2(x)
    assert_bytes(s, rs, "scales")
    assert_bytes(q, rq, "codes")


@pytest.mark.parametrize("seed", [0, 1234567, 2 ** 63 + 5])
def test_e5m2_stochastic_exhaustive_values(mx, seed):
    x = _exhaustive_blocks(step=8)
    note(f"quant_e5m2 stochastic exhaustive {x.shape} seed={seed}")
    q, s = run_quant(mx, x, seed=seed)
    rq, rs = O.grad_quant_e5m2(x, seed=seed)
    assert_bytes(s, rs, "scales")
    assert_bytes(q, rq, "codes")


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (41, 1536), (257, 1056), (1000, 2048)])
@pytest.mark.parametrize("seed", [None, 99])
def test_e5m2_ragged_shapes(mx, M, K, seed):
    x = synth.bf16_normal(np.random.default_rng(M + K), (M, K), std=1e-3, outlier_frac=0.02)
    note(f"quant_e5m2 M={M} K={K} seed={seed}")
    q, s = run_quant(mx, x, seed=seed)
    rq, rs = O.grad_quant_e5m2(x, seed=seed)
    assert_bytes(s, rs, "scales")
    assert_bytes(q, rq, "codes")


def test_e5m2_batched_stochastic_index_runs_over_batches(mx):
    B, M, K = 3, 40, 96
    x = synth.bf16_normal(np.random.default_rng(8), (B, M, K), std=1e-2)
    xd = dev_bf16(x)
    q = torch.empty((B, M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((B, M, K // 32), dtype=torch.uint8, device="cuda")
    note("quant_e5m2 batched stochastic")
    mx.mx_quant_e5m2(xd, q, s, seed=31)
    torch.cuda.synchronize()
    rq, rs = O.grad_quant_e5m2(x, seed=31)
    assert_bytes(host_u8(q), rq, "codes")
    assert_bytes(host_u8(s), rs, "scales")


@pytest.mark.parametrize("R,C", [(32, 8), (64, 64), (96, 40), (160, 72), (128, 200), (2048, 1032)])
@pytest.mark.parametrize("fmt,seed", [("e4m3", None), ("e5m2", None), ("e5m2", 77)])
def test_quant_transpose_shapes(mx, R, C, fmt, seed):
    x = synth.bf16_normal(np.random.default_rng(R * 3 + C), (R, C), outlier_frac=0.02)
    note(f"quant_transpose {fmt} R={R} C={C} seed={seed}")
    q, s = run_transpose(mx, x, fmt, seed)
    if fmt == "e4m3":
        rq, rs = O.quant_transpose_e4m3(x)
    else:
        rq, rs = O.quant_transpose_e5m2(x, seed=seed)
    assert_bytes(s, rs, "scales")
    assert_bytes(q, rq, "codes")


def test_quant_transpose_e4m3_equals_act_quant_of_the_transpose(mx):
    x = synth.bf16_normal(synth.rng_for(21), (512, 384), outlier_frac=0.05)
    note("quant_transpose e4m3 vs act_quant of x^T")
    q, s = run_transpose(mx, x, "e4m3")
    xt = dev_bf16(np.ascontiguousarray(x.T))
    qa = torch.empty((384, 512), dtype=torch.uint8, device="cuda")
    sa = torch.empty((384, 16), dtype=torch.uint8, device="cuda")
    mx.mx_act_quant(xt, qa, sa)
    torch.cuda.synchronize()
    assert np.array_equal(q, host_u8(qa)) and np.array_equal(s, host_u8(sa))


def _e5m2_operand(M, K, seed):
    g = synth.bf16_normal(synth.rng_for(seed), (M, K), std=1e-3, outlier_frac=0.01)
    return O.grad_quant_e5m2(g, seed=seed)


def _e4m3_rows_operand(N, K, seed):
    w = synth.bf16_normal(synth.rng_for(seed), (K, N), std=0.05)     # transposed on quantizing
    return O.quant_transpose_e4m3(w)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (41, 33, 96), (129, 257, 160), (300, 520, 1024),
                                   (64, 2048, 4096)])
def test_gemm_e5m2_e4m3_against_oracle(mx, M, N, K):
    a, a_s = _e5m2_operand(M, K, M + 1)
    b, b_s = _e4m3_rows_operand(N, K, N + 2)
    c = poison_bf16((M, N))
    note(f"gemm e5m2_e4m3 {M}x{N}x{K}")
    mx.mx_gemm_e5m2_e4m3(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), c)
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    ref, S = O.gemm_ref(O.decode_e5m2_rows(a, a_s), O.decode_e4m3_rows(b, b_s))
    ok = O.within_tolerance(out, ref, S)
    assert ok.all(), f"{np.count_nonzero(~ok)} of {ok.size} outside the bound"


def test_gemm_e5m2_e4m3_batched(mx):
    B, M, N, K = 3, 70, 96, 192
    a = np.stack([_e5m2_operand(M, K, 40 + i)[0] for i in range(B)])
    a_s = np.stack([_e5m2_operand(M, K, 40 + i)[1] for i in range(B)])
    b = np.stack([_e4m3_rows_operand(N, K, 50 + i)[0] for i in range(B)])
    b_s = np.stack([_e4m3_rows_operand(N, K, 50 + i)[1] for i in range(B)])
    c = poison_bf16((B, M, N))
    note("gemm e5m2_e4m3 batched")
    mx.mx_gemm_e5m2_e4m3(dev_u8(a), dev_u8(a_s), dev_u8(b), dev_u8(b_s), c)
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    for i in range(B):
        ref, S = O.gemm_ref(O.decode_e5m2_rows(a[i], a_s[i]), O.decode_e4m3_rows(b[i], b_s[i]))
        assert O.within_tolerance(out[i], ref, S).all()


@pytest.mark.parametrize("M,N,K,stochastic,sampled", [(256, 512, 384, True, False),
                                                       (1024, 2048, 1024, True, False),
                                                       (4096, 7168, 2048, False, True)])
def test_linear_backward_pipeline(mx, M, N, K, stochastic, sampled):
    # y = x W^T; dX = dY W and dW = dY^T x from E5M2 gradients and transposed E4M3 operands,
    # every step on the GPU, against the oracle's pipeline.  The layer of the 4096x7168x2048
    # forward GEMM runs with round-to-nearest-even gradients (the oracle's stochastic stream over
    # 29 M elements takes half a minute per operand on the host).
    rng = synth.rng_for(M + N + K)
    x = synth.bf16_normal(rng, (M, K), outlier_frac=0.01)
    W = synth.bf16_normal(rng, (N, K), std=0.05)
    dY = synth.bf16_normal(rng, (M, N), std=1e-3)
    xd, Wd, dYd = dev_bf16(x), dev_bf16(W), dev_bf16(dY)
    u8 = dict(dtype=torch.uint8, device="cuda")
    gq, gs = torch.empty((M, N), **u8), torch.empty((M, N // 32), **u8)
    wq, ws_ = torch.empty((K, N), **u8), torch.empty((K, N // 32), **u8)
    gtq, gts = torch.empty((N, M), **u8), torch.empty((N, M // 32), **u8)
    xq, xs = torch.empty((K, M), **u8), torch.empty((K, M // 32), **u8)
    dX, dW = poison_bf16((M, K)), poison_bf16((N, K))
    nws = mx.mx_gemm_splitk_workspace_size(M, K, N)             # dX: M x K output, contraction N
    ws = torch.zeros(nws, **u8) if nws else None
    note(f"linear backward {M}x{N}x{K}")
    s1, s2 = (101, 202) if stochastic else (None, None)
    mx.mx_quant_e5m2(dYd, gq, gs, seed=s1)
    mx.mx_quant_transpose_e4m3(Wd, wq, ws_)
    mx.mx_gemm_e5m2_e4m3_splitk(gq, gs, wq, ws_, dX, ws)
    mx.mx_quant_transpose_e5m2(dYd, gtq, gts, seed=s2)
    mx.mx_quant_transpose_e4m3(xd, xq, xs)
    mx.mx_gemm_e5m2_e4m3(gtq, gts, xq, xs, dW)
    torch.cuda.synchronize()
    r_gq, r_gs = O.grad_quant_e5m2(dY, seed=s1)
    r_wq, r_ws = O.quant_transpose_e4m3(W)
    r_gtq, r_gts = O.quant_transpose_e5m2(dY, seed=s2)
    r_xq, r_xs = O.quant_transpose_e4m3(x)
    for got, want, what in ((gq, r_gq, "dY codes"), (gs, r_gs, "dY scales"), (wq, r_wq, "W^T codes"),
                            (ws_, r_ws, "W^T scales"), (gtq, r_gtq, "dY^T codes"),
                            (gts, r_gts, "dY^T scales"), (xq, r_xq, "x^T codes"),
                            (xs, r_xs, "x^T scales")):
        assert_bytes(host_u8(got), want, what)
    for out_t, (aq, as_, bq, bs_), rows_n in ((dX, (r_gq, r_gs, r_wq, r_ws), M),
                                              (dW, (r_gtq, r_gts, r_xq, r_xs), N)):
        out = host_bf16_bits(out_t)
        A, B = O.decode_e5m2_rows(aq, as_), O.decode_e4m3_rows(bq, bs_)
        if sampled:
            rr = np.random.default_rng(3)
            rows, cols = rr.integers(0, rows_n, 3000), rr.integers(0, K, 3000)
            ref, S = O.gemm_ref_at(A, B, rows, cols)
            assert O.within_tolerance(out[rows, cols], ref, S).all()
            assert np.isfinite(O.bf16_to_f64(out)).all()
        else:
            ref, S = O.gemm_ref(A, B)
            assert O.within_tolerance(out, ref, S).all()
