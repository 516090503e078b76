"""Pins for the oracle's residual and GELU epilogues (CPU only).

* gelu_f64 against what fixes it apart from its own erfc call: textbook values of the normal CDF,
  the odd-part identity gelu(x) - gelu(-x) = x, the 1 + erf form from Python's math library
  where that form has no cancellation, the tail from math.erfc, and the Lipschitz constant from
  the closed form of the derivative's maximum.
* gemm_residual_ref is recomputed for tiny problems with exact rationals from raw bytes.
* gelu_within is tested on constructed values at its boundary.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx_oracle as O
from block_scaled_precision_act_amd import synth

# Standard normal CDF at 1, -1, 2 and -3 (textbook table values, 16 significant digits).
PHI = {1.0: 0.8413447460685429, -1.0: 0.1586552539314571, 2.0: 0.9772498680518208,
       -3.0: 0.001349898031630095}


@pytest.mark.parametrize("x", sorted(PHI))
def test_gelu_textbook_values(x):
    assert O.gelu_f64(x) == pytest.approx(x * PHI[x], rel=2e-15)


def test_gelu_zero_and_signed_zero():
    assert O.gelu_f64(0.0) == 0.0 and not np.signbit(O.gelu_f64(0.0))
    assert np.signbit(O.gelu_f64(-0.0))


def test_gelu_odd_part_identity():
    x = np.linspace(-12, 12, 48001)
    d = O.gelu_f64(x) - O.gelu_f64(-x)
    assert np.all(np.abs(d - x) <= 4e-16 * np.maximum(np.abs(x), 1))


def test_gelu_against_math_erf_where_it_does_not_cancel():
    x = np.linspace(-2.5, 6, 8501)
    want = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    assert np.allclose(O.gelu_f64(x), want, rtol=1e-14, atol=0)


def test_gelu_tail_against_math_erfc():
    x = -np.linspace(3, 37, 341)
    want = np.array([0.5 * v * math.erfc(-v / math.sqrt(2.0)) for v in x])
    assert np.allclose(O.gelu_f64(x), want, rtol=1e-13, atol=0)
    assert O.gelu_f64(-10.0) == pytest.approx(-7.619853024160527e-23, rel=1e-13)
    assert O.gelu_f64(40.0) == 40.0


def test_gelu_lipschitz_constant():
    # d/dx x Phi(x) = Phi(x) + x phi(x) is largest at x = sqrt 2 (where its derivative
    # phi(x) (2 - x^2) vanishes); the numeric slope never exceeds the stated constant.
    x = np.linspace(-8, 8, 1600001)
    slope = np.diff(O.gelu_f64(x)) / np.diff(x)
    r2 = math.sqrt(2.0)
    closed = 0.5 * math.erfc(-1.0) + r2 * math.exp(-1.0) / math.sqrt(2 * math.pi)
    assert closed <= O.GELU_LIPSCHITZ < 2.0
    assert np.abs(slope).max() <= O.GELU_LIPSCHITZ
    assert np.abs(slope).max() > closed - 1e-6


@pytest.mark.parametrize("a_kind,b_kind", [("fp8", "fp4"), ("fp8", "fp8"), ("fp4", "fp4")])
def test_residual_ref_exact_on_tiny_problems(a_kind, b_kind):
    w = synth.gemm_inputs(a_kind, b_kind, 3, 5, 64, seed=31, with_bias=True)
    dec_a = O.decode_fp4_rows if a_kind == "fp4" else O.decode_e4m3_rows
    dec_b = O.decode_fp4_rows if b_kind == "fp4" else O.decode_fp8_block
    A, B = dec_a(w.a, w.a_s), dec_b(w.b, w.b_s)
    res = synth.bf16_normal(np.random.default_rng(7), (3, 5))
    ref, S = O.gemm_residual_ref(A, B, O.bf16_to_f64(w.bias), res)
    bias = O.bf16_to_f64(w.bias)
    rv = O.bf16_to_f64(res)
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(64))
            exact += Fraction(float(bias[n])) + Fraction(float(rv[m, n]))
            assert abs(Fraction(float(ref[m, n])) - exact) <= Fraction(float(S[m, n])) * 2 ** -50 \
                + abs(exact) * 2 ** -52


def test_residual_ref_without_residual_is_gemm_ref():
    w = synth.gemm_inputs("fp8", "fp8", 4, 6, 96, seed=3, with_bias=True)
    A, B = O.decode_e4m3_rows(w.a, w.a_s), O.decode_fp8_block(w.b, w.b_s)
    r1, S1 = O.gemm_residual_ref(A, B, O.bf16_to_f64(w.bias))
    r2, S2 = O.gemm_ref(A, B, O.bf16_to_f64(w.bias))
    assert np.array_equal(r1, r2) and np.array_equal(S1, S2)


def test_gelu_ref_applies_gelu_to_the_biased_sum():
    w = synth.gemm_inputs("fp8", "fp4", 4, 6, 64, seed=4, with_bias=True)
    A, B = O.decode_e4m3_rows(w.a, w.a_s), O.decode_fp4_rows(w.b, w.b_s)
    g, pre, S = O.gemm_gelu_ref(A, B, O.bf16_to_f64(w.bias))
    want = (A @ B.T) + O.bf16_to_f64(w.bias)[None, :]
    assert np.allclose(pre, want, rtol=1e-15, atol=0)
    assert np.array_equal(g, O.gelu_f64(pre))


def _bits(v):
    return (np.array([v], np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_gelu_within_boundary():
    pre, g = 1.0, O.gelu_f64(1.0)
    v = 0.8515625                                    # a bf16 value, 0.0102 above gelu(1)
    gap = v - g
    rel = math.ldexp(abs(g), -7) + 2.0 ** -126
    assert gap > rel
    assert not O.gelu_within(_bits(v), np.array([pre]), np.array([0.0]))[0]
    S_edge = (gap - rel) * 2 ** 19
    assert O.gelu_within(_bits(v), np.array([pre]), np.array([S_edge * (1 + 1e-9)]))[0]
    assert not O.gelu_within(_bits(v), np.array([pre]), np.array([S_edge * (1 - 1e-6)]))[0]
    nan = np.array([0x7FC0], np.uint16)
    assert not O.gelu_within(nan, np.array([pre]), np.array([1e30]))[0]
    # a value whose GELU lies below the bf16 normal range is accepted as zero
    assert O.gelu_within(np.array([0x8000], np.uint16), np.array([-14.0]), np.array([0.0]))[0]
