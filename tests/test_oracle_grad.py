"""Pins for the oracle's backward-pass operands (CPU only).

* E5M2 decode against torch's float8_e5m2 cast (a library routine) for every finite code, and the
  round-to-nearest-even encode against torch's float32 -> float8_e5m2 cast over every bf16 value
  times every scale the gradient quantizer can meet.
* The scale rule against exact rationals for every positive finite bf16 amax, its floor and the
  E8M0 clamp.
* Philox4x64-10 against numpy's Philox bit generator (an independent implementation of the
  published algorithm), and the per-element index -> 32-bit word mapping against numpy's output
  stream.
* Stochastic rounding: the result is always one of the two neighbouring E5M2 values, values on
  the grid never move, the threshold sits exactly at u = ceil(2^32 * fraction), and the mean over
  many seeds is the input (unbiased) within its binomial error.
* Quantize-transpose puts the 32-blocks along the rows of the input (the contraction dimension
  of the GEMM that reads it).
* The backward GEMM references stay within the quantization error of the float64 product.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mx_oracle as O
from block_scaled_precision_act_amd import synth


def _finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def test_e5m2_decode_matches_torch_for_every_finite_code():
    codes = np.array([c for c in range(256) if c not in O.E5M2_SPECIAL], dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy().astype(np.float64)
    got = O.e5m2_to_f64(codes)
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    assert O.e5m2_to_f64(np.array([0x7B], np.uint8))[0] == O.E5M2_MAX
    for c in (0x7C, 0x7F, 0xFC, 0xFF):
        with pytest.raises(O.OracleRefusal):
            O.e5m2_to_f64(np.array([c], np.uint8))


def test_e5m2_rne_matches_torch_over_every_bf16_times_every_scale():
    b = _finite_bf16()
    v = O.bf16_to_f64(b)
    ys = []
    for E in range(-133, 114, 3):             # every third exponent: 83 scales x 65280 values
        y = v / 2.0 ** E
        ys.append(y[np.abs(y) <= O.E5M2_MAX])
    y = np.concatenate(ys)
    want = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    exact32 = y.astype(np.float32).astype(np.float64) == y       # torch casts from float32
    got = O.e5m2_encode_rne(y)
    assert np.array_equal(got[exact32], want[exact32])
    # the rest underflow float32: far below half the least E5M2 subnormal, a signed zero
    rest = ~exact32
    assert np.all(np.abs(y[rest]) < 2.0 ** -17)
    assert np.array_equal(got[rest], np.where(np.signbit(y[rest]), 0x80, 0x00).astype(np.uint8))


def test_grad_scale_rule_exact_for_every_bf16_amax():
    b = _finite_bf16()
    v = O.bf16_to_f64(b)
    b, v = b[v > 0], v[v > 0]
    x = np.zeros((len(b), 32), np.uint16)
    x[:, 7] = b
    E = O.grad_scale_bytes(x)[:, 0].astype(int) - 127
    floor = Fraction(2) ** -126
    for val, e in zip(v[::9], E[::9]):
        a = max(Fraction(float(val)), floor)
        need = Fraction(57344) * Fraction(2) ** int(e)
        lower = Fraction(57344) * Fraction(2) ** (int(e) - 1)
        assert (a <= need and (e == -127 or not a <= lower)), (val, e)
    assert E.min() == -127 and E.max() == 113
    zero = np.zeros((1, 32), np.uint16)
    assert O.grad_scale_bytes(zero)[0, 0] == 0


@pytest.mark.parametrize("key,start", [(0, 0), (42, 1), (1234, 2 ** 32 - 1), (2 ** 64 - 1, 2 ** 63)])
def test_philox_matches_numpy(key, start):
    cnt = np.array([start - 1 if start else 2 ** 64 - 1] + ([0, 0, 0] if start else [2 ** 64 - 1] * 3),
                   dtype=np.uint64)
    bg = np.random.Philox(key=np.array([key, 0], dtype=np.uint64), counter=cnt)
    raw = bg.random_raw(4 * 6)
    ctr = np.arange(start, start + 6, dtype=np.uint64)
    z = np.zeros_like(ctr)
    w = O.philox4x64_10((ctr, z, z, z), (np.uint64(key), np.uint64(0)))
    assert np.array_equal(np.stack(w, axis=1).reshape(-1), raw)


def test_uniform_u32_is_the_philox_stream_in_32_bit_halves():
    seed = 987654321
    bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                          counter=np.array([2 ** 64 - 1] * 4, dtype=np.uint64))
    raw = bg.random_raw(400)                                   # blocks 0..99, 4 words each
    halves = np.stack([raw & 0xFFFFFFFF, raw >> 32], axis=1).reshape(-1)
    got = O.uniform_u32(seed, np.arange(800, dtype=np.uint64))
    assert np.array_equal(got, halves)


def _grid():
    return O.e5m2_to_f64(np.arange(0x7C, dtype=np.uint8))


def test_stochastic_result_is_a_neighbour_and_grid_values_stay():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-O.E5M2_MAX, O.E5M2_MAX, 20000),
                        rng.normal(0, 1e-4, 20000), _grid(), -_grid()])
    u = rng.integers(0, 2 ** 32, y.size, dtype=np.uint64)
    got = O.e5m2_to_f64(O.e5m2_encode_stochastic(y, u))
    g = _grid()
    a = np.abs(y)
    lo = g[np.searchsorted(g, a, side="right") - 1]
    hi = g[np.minimum(np.searchsorted(g, a, side="right"), len(g) - 1)]
    ok = (np.abs(got) == lo) | (np.abs(got) == hi)
    assert ok.all()
    on = np.isin(a, g)
    assert np.array_equal(np.abs(got[on]), a[on])
    assert np.array_equal(np.signbit(got), np.signbit(y))


def test_stochastic_threshold_is_exact():
    # y = 1 + 1/8 + 1/32 between 1 and 1.25: fraction 0.625 -> threshold 0.625 * 2^32
    y = np.array([1.0 + 1 / 8 + 1 / 32])
    t = int(0.625 * 2 ** 32)
    assert O.e5m2_to_f64(O.e5m2_encode_stochastic(y, [t - 1]))[0] == 1.25
    assert O.e5m2_to_f64(O.e5m2_encode_stochastic(y, [t]))[0] == 1.0
    # a value a hair above an E5M2 subnormal: fraction 2^-20 of the 2^-16 step
    y = np.array([3 * 2.0 ** -16 + 2.0 ** -36])
    assert O.e5m2_to_f64(O.e5m2_encode_stochastic(y, [2 ** 12 - 1]))[0] == 4 * 2.0 ** -16
    assert O.e5m2_to_f64(O.e5m2_encode_stochastic(y, [2 ** 12]))[0] == 3 * 2.0 ** -16


@pytest.mark.parametrize("y", [1.1, -3.3e-5, 0.3 * 2.0 ** -16, 40000.0, 7.77])
def test_stochastic_rounding_is_unbiased(y):
    n = 20000
    u = O.uniform_u32(777, np.arange(n, dtype=np.uint64))
    got = O.e5m2_to_f64(O.e5m2_encode_stochastic(np.full(n, y), u))
    g = _grid()
    a = abs(y)
    lo = g[np.searchsorted(g, a, side="right") - 1]
    hi = g[np.searchsorted(g, a, side="right")]
    p = (a - lo) / (hi - lo)
    sigma = (hi - lo) * np.sqrt(p * (1 - p) / n)
    assert abs(np.abs(got).mean() - a) <= 5 * sigma + 1e-300


def test_grad_quant_rne_within_half_an_e5m2_step_and_never_clipped():
    x = synth.bf16_normal(synth.rng_for(3), (64, 256), outlier_frac=0.05)
    q, s = O.grad_quant_e5m2(x)
    deq = O.decode_e5m2_rows(q, s)
    v = O.bf16_to_f64(x)
    # normal E5M2 values are within 2^-3 of the value, subnormals within 2^-17 * 2^E
    E = np.repeat(s.astype(np.int64) - 127, 32, axis=-1)
    assert np.all(np.abs(deq - v) <= np.ldexp(np.abs(v), -3) + np.ldexp(1.0, E - 17))
    blocks = np.abs(v).reshape(64, 8, 32).max(axis=-1)
    assert np.all(blocks <= O.E5M2_MAX * np.ldexp(1.0, s.astype(np.int64) - 127))


def test_grad_quant_stochastic_draws_by_output_index():
    x = synth.bf16_normal(synth.rng_for(4), (8, 64))
    q1, s1 = O.grad_quant_e5m2(x, seed=5)
    q2, s2 = O.grad_quant_e5m2(x, seed=5)
    q3, _ = O.grad_quant_e5m2(x, seed=6)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2) and not np.array_equal(q1, q3)
    y = (O.bf16_to_f64(x).reshape(8, 2, 32) / O.e8m0_to_f64(s1)[..., None]).reshape(8, 64)
    u = O.uniform_u32(5, np.arange(8 * 64, dtype=np.uint64)).reshape(8, 64)
    assert np.array_equal(q1, O.e5m2_encode_stochastic(y, u))


def test_quant_transpose_blocks_run_along_the_input_rows():
    R, C = 64, 96
    x = synth.bf16_normal(synth.rng_for(5), (R, C))
    x[3, 10] = 0x4700                                    # 32768: dominates column 10, rows 0..31
    q, s = O.quant_transpose_e4m3(x)
    assert q.shape == (C, R) and s.shape == (C, R // 32)
    big = s[10, 0]
    assert big > s[10, 1] and big > s[11, 0]            # only column 10's first row block moved
    qa, sa = O.act_quant(np.ascontiguousarray(x.T))
    assert np.array_equal(q, qa) and np.array_equal(s, sa)
    qt, st = O.quant_transpose_e5m2(x, seed=9)
    qg, sg = O.grad_quant_e5m2(np.ascontiguousarray(x.T), seed=9)
    assert np.array_equal(qt, qg) and np.array_equal(st, sg)


def test_backward_references_within_quantization_error():
    # y = x W^T: dX = dY W and dW = dY^T x, from E5M2 gradients and E4M3 transposed operands.
    M, N, K = 64, 96, 128
    rng = synth.rng_for(6)
    x = synth.bf16_normal(rng, (M, K))
    W = synth.bf16_normal(rng, (N, K), std=0.05)
    dY = synth.bf16_normal(rng, (M, N), std=1e-3)
    gq, gs = O.grad_quant_e5m2(dY, seed=11)                    # [M, N], blocks along N
    wq, ws = O.quant_transpose_e4m3(W)                          # [K, N], blocks along N
    dX, S = O.gemm_ref(O.decode_e5m2_rows(gq, gs), O.decode_e4m3_rows(wq, ws))
    gtq, gts = O.quant_transpose_e5m2(dY, seed=12)              # [N, M], blocks along M
    xq, xs = O.quant_transpose_e4m3(x)                          # [K, M], blocks along M
    dW, S2 = O.gemm_ref(O.decode_e5m2_rows(gtq, gts), O.decode_e4m3_rows(xq, xs))
    dYf, Wf, xf = O.bf16_to_f64(dY), O.bf16_to_f64(W), O.bf16_to_f64(x)
    exact_dX, exact_dW = dYf @ Wf, dYf.T @ xf
    # each E5M2 value is within 2^-2 of its input (stochastic: a neighbour), each E4M3 within 2^-4
    assert np.all(np.abs(dX - exact_dX) <= (2.0 ** -2 + 2.0 ** -4 + 2.0 ** -6) * (np.abs(dYf) @ np.abs(Wf)) + 1e-30)
    assert np.all(np.abs(dW - exact_dW) <= (2.0 ** -2 + 2.0 ** -4 + 2.0 ** -6) * (np.abs(dYf).T @ np.abs(xf)) + 1e-30)
    assert dX.shape == (M, K) and dW.shape == (N, K)
