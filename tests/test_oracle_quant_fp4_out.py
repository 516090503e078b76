"""Pins for the oracle's MXFP4-quantized GEMM output (CPU only).

* The E2M1 error bound used by quant_fp4_output_within is checked against every E2M1 value and
  every midpoint between neighbours (the worst cases of round-to-nearest).
* gemm_quant_fp4_ref is recomputed for tiny problems with exact rationals and a brute-force
  nearest-value search over the printed FP4 table.
* The acceptance predicate is tested at its boundary.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx_oracle as O
from block_scaled_precision_act_amd import synth

TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_rounding_error_bound_is_tight_and_valid():
    # worst case of nearest rounding: the midpoints; |q - v| <= v / 4 + 1/4 for every v in [0, 6]
    v = np.linspace(0, 6, 60001)
    q = O.e2m1_to_f64(O.e2m1_encode_rne(v))
    assert np.all(np.abs(q - v) <= v / 4 + 0.25 + 1e-15)
    mids = np.array([(a + b) / 2 for a, b in zip(TABLE, TABLE[1:])])
    err = np.abs(O.e2m1_to_f64(O.e2m1_encode_rne(mids)) - mids)
    assert np.isclose(err.max(), 1.0)                       # the midpoint 5 of 4 and 6 goes to 4
    assert np.all(err <= mids / 4 + 0.25)


@pytest.mark.parametrize("gelu", [False, True])
def test_gemm_quant_fp4_ref_exact_on_tiny_problems(gelu):
    w = synth.gemm_inputs("fp4", "fp4", 2, 64, 64, seed=21, with_bias=True)
    A, B = O.decode_fp4_rows(w.a, w.a_s), O.decode_fp4_rows(w.b, w.b_s)
    bias = O.bf16_to_f64(w.bias)
    ref, S, y, packed, sb = O.gemm_quant_fp4_ref(A, B, bias, gelu=gelu)
    for m in range(2):
        for n in range(64):
            exact = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(64))
            exact += Fraction(float(bias[n]))
            if not gelu:
                assert abs(Fraction(float(ref[m, n])) - exact) <= Fraction(float(S[m, n])) * 2 ** -50
            else:   # GELU of the exact pre-activation, x Phi(x) with Python's math.erfc
                x = float(exact)
                g = 0.5 * x * math.erfc(-x / math.sqrt(2.0))
                assert abs(ref[m, n] - g) <= 1e-12 * abs(g) + 1e-300
            # y is the bf16 value nearest the (GELU'd) sum: within half a bf16 spacing of it
            target = float(exact) if not gelu else g
            # (below the bf16 range, half the least subnormal: 2^-134)
            assert abs(O.bf16_to_f64(y[m, n]) - target) <= 2.0 ** -8 * abs(target) + 2.0 ** -134
    # codes: the nearest table value of y / 2^E, by brute force
    yv = O.bf16_to_f64(y)
    codes = O.fp4_unpack(packed)
    E = np.repeat(sb.astype(np.int64) - 127, 32, axis=-1)
    for m in range(2):
        for n in range(64):
            t = yv[m, n] / 2.0 ** E[m, n]
            d = [abs(abs(t) - x) for x in TABLE]
            best = min(d)
            cands = [i for i, di in enumerate(d) if di == best]
            c = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
            assert (codes[m, n] & 7) == c


def test_quant_fp4_output_within_boundary():
    # one block: ref = 5 (y = 5 exactly, t = 0) -> q = 4 or 6 at scale 2^0 (amax 5 -> E = 0)
    packed = np.zeros((1, 16), np.uint8)
    sb = np.full((1, 1), 127, np.uint8)
    ref = np.zeros((1, 32))
    ref[0, 0] = 5.0
    packed[0, 0] = 7                                        # element 0 -> 6.0
    ok = O.quant_fp4_output_within(packed, sb, ref, np.zeros((1, 32)))
    assert ok[0, 0]                                        # |6 - 5| = 1 <= 5/4 + 1/4
    packed[0, 0] = 5                                        # element 0 -> 3.0: |3 - 5| = 2 > 1.5
    ok = O.quant_fp4_output_within(packed, sb, ref, np.zeros((1, 32)))
    assert not ok[0, 0]
    t = np.zeros((1, 32))
    t[0, 0] = 0.4                                           # 5/4 + 0.4/4 + 0.4 + 1/4 = 2.0
    assert O.quant_fp4_output_within(packed, sb, ref, t)[0, 0]
    t[0, 0] = 0.39
    assert not O.quant_fp4_output_within(packed, sb, ref, t)[0, 0]


def test_quant_fp4_output_within_uses_each_blocks_scale():
    # two blocks of one row with scales 2^0 and 2^4: a value in block 1 is checked against its own scale
    packed = np.zeros((1, 32), np.uint8)
    sb = np.array([[127, 131]], np.uint8)
    ref = np.zeros((1, 64))
    ref[0, 32] = 3.0                       # decodes to 0 at scale 16: |0 - 3| = 3 <= 16 / 4 + 3 / 4
    assert O.quant_fp4_output_within(packed, sb, ref, np.zeros((1, 64)))[0, 32]
    ref[0, 0] = 3.0                        # the same at scale 1: |0 - 3| = 3 > 1 / 4 + 3 / 4
    assert not O.quant_fp4_output_within(packed, sb, ref, np.zeros((1, 64)))[0, 0]
