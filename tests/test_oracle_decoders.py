"""Pins for the oracle's decoders (CPU only).

Each decoder is checked against something other than itself: the table and constants printed on
the formats.py page (tests/golden/formats_page.json), an independent bit-field derivation, the
closed form 2^(b-127), and torch's float8_e4m3fn -> float32 cast (a library routine; the
formats.py page decodes E4M3 with the same cast).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mx_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "formats_page.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_constants_match_page(golden):
    assert O.FP8_MAX == golden["fp8_max"]
    assert O.BLOCK == golden["block"]
    assert O.E8M0_NAN == golden["e8m0_nan"]
    assert tuple(O.E4M3_NAN) == tuple(golden["e4m3_nan"])


def test_fp4_table_matches_printed_table(golden):
    got = O.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    want = np.array(golden["fp4_table"])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.signbit(got[golden["fp4_negative_zero_code"]]) and got[8] == 0.0


def test_fp4_table_from_bit_fields():
    # E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        want = math.copysign(mag, -1.0 if s else 1.0)
        got = float(O.e2m1_to_f64(np.uint8(c)))
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c


def test_e8m0_closed_form_all_bytes():
    b = np.arange(255, dtype=np.uint8)
    got = O.e8m0_to_f64(b)
    for i in range(255):
        assert got[i] == math.ldexp(1.0, i - 127)
    assert got[0] == 2.0 ** -127 and got[127] == 1.0 and got[254] == 2.0 ** 127


def test_e8m0_nan_refused():
    with pytest.raises(O.OracleRefusal):
        O.e8m0_to_f64(np.array([127, 255], dtype=np.uint8))


def test_e4m3_decode_all_codes_vs_torch_cast():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    got = O.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_e4m3_decode_known_points(golden):
    bias = golden["e4m3_exponent_bias"]
    pts = {0x38: 1.0, 0x7E: golden["fp8_max"], 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
           0x08: 2.0 ** (1 - bias), 0xB8: -1.0, 0xFE: -448.0, 0x40: 2.0}
    for c, v in pts.items():
        assert float(O.e4m3_to_f64(np.uint8(c))) == v, hex(c)
    z = O.e4m3_to_f64(np.array([0x00, 0x80], dtype=np.uint8))
    assert z[0] == 0 and not np.signbit(z[0]) and z[1] == 0 and np.signbit(z[1])
    assert np.max(O.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))) == 448.0


@pytest.mark.parametrize("code", [0x7F, 0xFF])
def test_e4m3_nan_refused(code):
    with pytest.raises(O.OracleRefusal):
        O.e4m3_to_f64(np.array([0x38, code], dtype=np.uint8))


def test_fp4_unpack_low_nibble_first(golden):
    fx = golden["fp4_packing"]
    codes = O.fp4_unpack(np.array([[fx["byte"]]], dtype=np.uint8))
    assert codes.tolist() == [fx["codes_low_nibble_first"]]
    rng = np.random.default_rng(0)
    p = rng.integers(0, 256, size=(3, 16)).astype(np.uint8)
    c = O.fp4_unpack(p)
    for r in range(3):
        for j in range(16):
            assert c[r, 2 * j] == p[r, j] % 16 and c[r, 2 * j + 1] == p[r, j] // 16


def test_decode_fp4_rows_scale_per_row_block():
    rng = np.random.default_rng(1)
    R, K = 3, 96
    packed = rng.integers(0, 256, size=(R, K // 2)).astype(np.uint8)
    scales = rng.integers(100, 150, size=(R, K // 32)).astype(np.uint8)
    got = O.decode_fp4_rows(packed, scales)
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(R):
        for k in range(K):
            byte = int(packed[r, k // 2])
            code = byte & 15 if k % 2 == 0 else byte >> 4
            v = table[code & 7] * (-1 if code & 8 else 1)
            assert got[r, k] == v * 2.0 ** (int(scales[r, k // 32]) - 127)


def test_decode_fp8_block_ragged_rows():
    rng = np.random.default_rng(2)
    N, K = 70, 96            # 3 x 3 scale blocks, the last block-row only 6 rows tall
    codes = rng.integers(0, 0x7F, size=(N, K)).astype(np.uint8)
    scales = rng.integers(110, 140, size=(3, 3)).astype(np.uint8)
    got = O.decode_fp8_block(codes, scales)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for n in range(N):
        for k in range(K):
            assert got[n, k] == ref[n, k] * 2.0 ** (int(scales[n // 32, k // 32]) - 127)
    with pytest.raises(O.OracleRefusal):
        O.decode_fp8_block(codes, scales[:2])


def test_decode_shape_refusals():
    with pytest.raises(O.OracleRefusal):
        O.decode_fp4_rows(np.zeros((2, 8), np.uint8), np.zeros((2, 1), np.uint8))   # K = 16
    with pytest.raises(O.OracleRefusal):
        O.decode_fp4_rows(np.zeros((2, 16), np.uint8), np.zeros((2, 2), np.uint8))  # wrong scale
    with pytest.raises(O.OracleRefusal):
        O.decode_e4m3_rows(np.zeros((2, 64), np.uint8), np.zeros((2, 1), np.uint8))


def test_bf16_widening_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(bits)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(t)
    assert np.array_equal(v[fin], t[fin])
    assert np.array_equal(np.isnan(v), np.isnan(t))
