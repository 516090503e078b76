"""Pins for the oracle's quantized GEMM output (CPU only).

* f64_to_bf16_rne, the bf16 rounding of an exact value, is checked against what fixes it: every
  finite bf16 value rounds to itself, every midpoint of two neighbours goes to the even one and
  anything off the midpoint to the nearer one (all 32,639 positive neighbour pairs, both signs),
  and on float32 inputs it agrees with torch's float32 -> bfloat16 cast (a library rounding).
* gemm_act_quant_ref is recomputed for tiny problems with exact rationals and a brute-force
  search for the nearest bf16 value.
* quant_output_within is tested on constructed values at its boundary.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mx_oracle as O
from block_scaled_precision_act_amd import synth


def _finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_every_finite_bf16_rounds_to_itself():
    bits = _finite_bf16()
    assert np.array_equal(O.f64_to_bf16_rne(O.bf16_to_f64(bits)), bits)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_midpoints_go_to_even_and_off_midpoints_to_nearer(sign):
    pos = np.arange(0x0000, 0x7F80, dtype=np.uint16)          # +0 .. largest finite, increasing
    v = O.bf16_to_f64(pos)
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2                                         # exact in float64
    want_even = np.where((pos[:-1] & 1) == 0, pos[:-1], pos[1:])
    sgn = np.uint16(0x8000) if sign < 0 else np.uint16(0)
    assert np.array_equal(O.f64_to_bf16_rne(sign * mid), want_even | sgn)
    eps = (hi - lo) / 1024                                      # exact power-of-two fractions
    assert np.array_equal(O.f64_to_bf16_rne(sign * (mid - eps)), pos[:-1] | sgn)
    assert np.array_equal(O.f64_to_bf16_rne(sign * (mid + eps)), pos[1:] | sgn)


def test_agrees_with_torch_float32_to_bfloat16_cast():
    rng = np.random.default_rng(77)
    f = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0),
        (rng.random(100_000) * 2 - 1).astype(np.float32) * np.float32(2.0 ** -128),   # subnormal
        rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    f = f[np.isfinite(f) & (np.abs(f) < np.float32(3.3e38))]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_rne(f.astype(np.float64)), want)


def test_signed_zero_and_refusals():
    assert O.f64_to_bf16_rne(np.array([-0.0, 0.0, -1e-300, 1e-300])).tolist() == \
        [0x8000, 0x0000, 0x8000, 0x0000]
    for bad in (np.inf, np.nan, 3.5e38):
        with pytest.raises(O.OracleRefusal):
            O.f64_to_bf16_rne(np.array([bad]))


def _nearest_bf16_bits(r: Fraction) -> int:
    """Brute force: the finite bf16 pattern nearest to the rational r, ties to the even one."""
    bits = _finite_bf16()
    bits = bits[(bits & 0x8000) == (0x8000 if r < 0 else 0)]
    vals = O.bf16_to_f64(bits)
    order = np.argsort(vals)
    bits, vals = bits[order], vals[order]
    i = int(np.searchsorted(vals, float(r)))
    cands = [int(bits[j]) for j in (i - 1, i, i + 1) if 0 <= j < len(bits)]
    def key(bb):
        d = abs(Fraction(float(O.bf16_to_f64(np.array([bb], np.uint16))[0])) - r)
        return (d, bb & 1)
    return min(cands, key=key)


@pytest.mark.parametrize("b_kind", ["fp4", "fp8"])
def test_gemm_act_quant_ref_brute_force(b_kind):
    w = synth.gemm_inputs("fp8", b_kind, 3, 64, 96, seed=2024, with_bias=True)
    A = O.decode_e4m3_rows(w.a, w.a_s)
    B = O.decode_fp4_rows(w.b, w.b_s) if b_kind == "fp4" else O.decode_fp8_block(w.b, w.b_s)
    bias = O.bf16_to_f64(w.bias)
    ref, S, y, codes, scales = O.gemm_act_quant_ref(A, B, bias)
    for m in range(3):
        for n in range(0, 64, 7):
            exact = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(96)) \
                + Fraction(float(bias[n]))
            assert y[m, n] == _nearest_bf16_bits(exact), (m, n)
    c2, s2 = O.act_quant(y)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    assert O.quant_output_within(codes, scales, ref, S).all()


def test_quant_output_within_boundary():
    # One 32-block, scale byte 127 (2^0); ref = 100 with S = 100: t = 100/128 + 100/2^20.
    scales = np.array([[127]], dtype=np.uint8)
    ref = np.full((1, 32), 100.0)
    S = np.full((1, 32), 100.0)
    t = 100 / 128 + 100 / 2 ** 20
    bound = (100 + t) / 16 + t + 2.0 ** -10
    codes = O.e4m3_encode_rne(np.full((1, 32), 96.0))          # 96 = 100 - 4, an E4M3 value
    assert O.quant_output_within(codes, scales, ref, S).all() == (4 <= bound)
    codes_far = O.e4m3_encode_rne(np.full((1, 32), 112.0))     # 12 away: beyond the bound
    assert 12 > bound and not O.quant_output_within(codes_far, scales, ref, S).any()
    # Every term counts: at ref = S = 102.8 the code for 96 is 6.8 away, inside the bound (7.28)
    # only with the GEMM term t added on its own as well as inside 2^-4 (|ref| + t).
    ref2 = np.full((1, 32), 102.8)
    t2 = 102.8 / 128 + 102.8 / 2 ** 20
    assert (102.8 + t2) / 16 + 2.0 ** -10 < 6.8 < (102.8 + t2) / 16 + t2 + 2.0 ** -10
    assert O.quant_output_within(codes, scales, ref2, ref2).all()
    # The subnormal term: ref 0, S 0 -> bound 2^(E-10); code 1 is 2^-9 * 2^E, beyond it.
    z = np.zeros((1, 32))
    one = np.ones((1, 32), dtype=np.uint8)
    assert not O.quant_output_within(one, scales, z, z).any()
    assert O.quant_output_within(np.zeros((1, 32), np.uint8), scales, z, z).all()


def test_quant_output_within_explicit_t():
    # ref 100, code for 112 at scale 2^0: 12 away; bound = (100 + t) / 16 + t + 2^-10 reaches 12
    # at t = (12 - 6.25 - 2^-10) * 16 / 17 = 5.41085 (the GELU bound is passed this way).
    scales = np.array([[127]], dtype=np.uint8)
    ref = np.full((1, 32), 100.0)
    codes = O.e4m3_encode_rne(np.full((1, 32), 112.0))
    assert O.quant_output_within(codes, scales, ref, None, t=np.full((1, 32), 5.42)).all()
    assert not O.quant_output_within(codes, scales, ref, None, t=np.full((1, 32), 5.40)).any()
    # the default t is the GEMM bound: S = 0 gives t = 100/128, far below 5.4
    assert not O.quant_output_within(codes, scales, ref, np.zeros((1, 32))).any()


def test_gelu_output_bound_terms():
    g = np.array([0.0, 128.0, 0.0, -256.0])
    S = np.array([0.0, 0.0, 2.0 ** 19, 0.0])
    assert np.array_equal(O.gelu_output_bound(g, S),
                          [2.0 ** -126, 1.0 + 2.0 ** -126, 1.0 + 2.0 ** -126, 2.0 + 2.0 ** -126])
