"""Pins for the oracle's MXFP4 activation producer (CPU only).

* The scale rule against exact rationals for every positive finite bf16 amax (and the float32
  floor): E is the smallest integer with amax <= 6 * 2^E.
* The E2M1 encode against a brute-force nearest-value search written here from the printed
  table, over every bf16 value in [-6, 6]; the midpoints of neighbouring values go to the even
  code; the sign of zero is kept.
* The packing order (element 2j in the low nibble) against the decoder's unpacking.
* End to end: every quantized value is the nearest E2M1 value of x / 2^E and the block maximum
  is not lost to clipping.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx_oracle as O
from block_scaled_precision_act_amd import synth

TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]        # "formats.py": FP4_TABLE, codes 0..7


def _bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint16)
    v = O.bf16_to_f64(bits)
    ok = np.isfinite(v)
    return bits[ok], v[ok]


def test_scale_rule_exact_for_every_bf16_amax():
    bits, v = _bf16_values()
    pos = (v > 0)
    bits, v = bits[pos], v[pos]
    x = np.zeros((len(bits), 32), dtype=np.uint16)
    x[:, 5] = bits
    got = O.act_scale_fp4_bytes(x)[:, 0].astype(int) - 127
    floor = Fraction(float(np.float32(1e-4)))
    for b, val, e in zip(bits[::7], v[::7], got[::7]):       # every 7th: 4.6k exact checks
        a = max(Fraction(float(val)), floor)
        assert a <= 6 * Fraction(2) ** int(e) and not a <= 6 * Fraction(2) ** (int(e) - 1), (b, e)
    # and all of them against the float64 form of the same rule
    a = np.maximum(v, float(np.float32(1e-4)))
    assert np.all(a <= 6 * np.ldexp(1.0, got)) and np.all(a > 6 * np.ldexp(1.0, got - 1))


def test_zero_block_uses_the_floor():
    x = np.zeros((1, 32), dtype=np.uint16)
    assert int(O.act_scale_fp4_bytes(x)[0, 0]) - 127 == -15       # 1e-4 <= 6 * 2^-15


def _nearest_code(y: float) -> int:
    a = abs(y)
    d = [abs(a - t) for t in TABLE]
    m = min(d)
    cands = [i for i, di in enumerate(d) if di == m]
    code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return code | (8 if np.signbit(y) else 0)


def test_encode_against_brute_force_on_every_bf16_in_range():
    _, v = _bf16_values()
    v = v[np.abs(v) <= 6.0]
    got = O.e2m1_encode_rne(v)
    want = np.array([_nearest_code(float(y)) for y in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_encode_midpoints_go_to_even_and_signs_are_kept():
    mids = [(a + b) / 2 for a, b in zip(TABLE[:-1], TABLE[1:])]
    got = O.e2m1_encode_rne(np.array(mids))
    assert [int(c) for c in got] == [0, 2, 2, 4, 4, 6, 6]
    assert int(O.e2m1_encode_rne(np.array([-0.0]))[0]) == 8
    assert int(O.e2m1_encode_rne(np.array([-0.1]))[0]) == 8
    assert [int(c) for c in O.e2m1_encode_rne(-np.array(TABLE))] == [8 + i for i in range(8)]
    with pytest.raises(O.OracleRefusal):
        O.e2m1_encode_rne(np.array([6.5]))


def test_pack_order_matches_the_decoder():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (7, 64), dtype=np.uint8)
    packed = O.fp4_pack(codes)
    assert packed.shape == (7, 32)
    assert np.array_equal(O.fp4_unpack(packed), codes)
    assert packed[0, 0] == (codes[0, 0] | (codes[0, 1] << 4))


def test_act_quant_fp4_end_to_end_properties():
    x = synth.bf16_normal(synth.rng_for(99), (64, 256), outlier_frac=0.02)
    packed, sb = O.act_quant_fp4(x)
    codes = O.fp4_unpack(packed)
    xv = O.bf16_to_f64(x).reshape(64, 8, 32)
    s = O.e8m0_to_f64(sb)[..., None]
    y = xv / s
    assert np.all(np.abs(y) <= 6.0)
    q = O.e2m1_to_f64(codes).reshape(64, 8, 32)
    # the nearest E2M1 value: no table value is strictly closer
    t = np.array(TABLE)
    best = np.min(np.abs(np.abs(y)[..., None] - t), axis=-1)
    assert np.all(np.abs(np.abs(q) - np.abs(y)) == best)
    # the block maximum lands in the top binade (3, 6] of E2M1 magnitudes: E is minimal
    amax = np.abs(xv).max(axis=-1)
    assert np.all(amax / s[..., 0] > 3.0)
