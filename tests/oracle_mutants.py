"""Planted mistakes for the oracle, one at a time: a pytest plugin for the mutation test.

Loaded with `-p oracle_mutants` and the environment variable ORACLE_MUTANT naming one entry of
MUTANTS, it replaces one function (or table) of oracle.mx_oracle, in the test process only, with
a copy that carries one plausible mistake: a dropped term, a wrong sign, index or bias, a wrong
rounding tie, a transposed operand.  tests/test_oracle_mutations.py runs the oracle's pin tests
under each mutant and requires that at least one of them fails, so that the pins are shown to
pin the oracle to something other than itself.  ORACLE_MUTANT=none changes nothing (the control
run, which must pass).  Nothing outside the tests loads this file.
"""
import os

import numpy as np


def _fp4_unpack_high_nibble_first(O):
    def fp4_unpack(packed):
        p = np.asarray(packed, dtype=np.uint8)
        codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
        codes[..., 0::2] = p >> 4                      # planted: high nibble first
        codes[..., 1::2] = p & 0x0F
        return codes
    O.fp4_unpack = fp4_unpack


def _fp4_table_typo(O):
    t = list(O.FP4_TABLE)
    t[5], t[13] = 2.5, -2.5                            # planted: 3.0 written as 2.5
    O.FP4_TABLE = tuple(t)


def _e8m0_bias_126(O):
    def e8m0_to_f64(scale_bytes):
        s = np.asarray(scale_bytes, dtype=np.uint8)
        if np.any(s == O.E8M0_NAN):
            raise O.OracleRefusal("NaN scale")
        return np.ldexp(1.0, s.astype(np.int64) - 126)  # planted: bias 126
    O.e8m0_to_f64 = e8m0_to_f64


def _e4m3_decode(O, bias=7, sub_exp=-9):
    def e4m3_to_f64(codes):
        b = np.asarray(codes, dtype=np.uint8)
        if np.any((b == 0x7F) | (b == 0xFF)):
            raise O.OracleRefusal("NaN code")
        sign = np.where(b >> 7, -1.0, 1.0)
        e = ((b >> 3) & 0xF).astype(np.int64)
        m = (b & 0x7).astype(np.float64)
        mag = np.where(e == 0, np.ldexp(m, sub_exp), np.ldexp(1.0 + m / 8.0, e - bias))
        return sign * mag
    return e4m3_to_f64


def _e4m3_bias_8(O):
    O.e4m3_to_f64 = _e4m3_decode(O, bias=8, sub_exp=-10)  # planted: exponent bias 8


def _e4m3_subnormal_step(O):
    O.e4m3_to_f64 = _e4m3_decode(O, sub_exp=-10)          # planted: subnormals m * 2^-10


def _fp8_block_scale_transposed(O):
    def decode_fp8_block(codes, scale_bytes):
        c = np.asarray(codes, dtype=np.uint8)
        N, K = c.shape
        s = np.asarray(scale_bytes, dtype=np.uint8)
        if s.shape != (-(-N // O.BLOCK), -(-K // O.BLOCK)):
            raise O.OracleRefusal("block scales do not cover the weight")
        scale = O.e8m0_to_f64(s)
        rows = np.arange(N) // O.BLOCK
        cols = np.arange(K) // O.BLOCK
        return O.e4m3_to_f64(c) * scale.T[rows[:, None], cols[None, :]]   # planted: [k/32][n/32]
    O.decode_fp8_block = decode_fp8_block


def _encode(tie_rule="even", keep_zero_sign=True):
    def e4m3_encode_rne(y, O):
        y = np.asarray(y, dtype=np.float64)
        grid = O.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
        a = np.abs(y)
        hi = np.minimum(np.searchsorted(grid, a, side="left"), len(grid) - 1)
        lo = np.maximum(hi - 1, 0)
        d_lo, d_hi = a - grid[lo], grid[hi] - a
        if tie_rule == "even":
            tie_hi = hi % 2 == 0
        elif tie_rule == "odd":
            tie_hi = hi % 2 == 1
        else:                                          # "away": ties go to the larger magnitude
            tie_hi = np.ones_like(hi, dtype=bool)
        pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & tie_hi)
        code = np.where(pick_hi, hi, lo)
        code = np.where(a == grid[hi], hi, code).astype(np.uint8)
        neg = np.signbit(y) if keep_zero_sign else (y < 0) & (code != 0)
        return code | np.where(neg, 0x80, 0).astype(np.uint8)
    return e4m3_encode_rne


def _set_encode(O, **kw):
    f = _encode(**kw)
    O.e4m3_encode_rne = lambda y: f(y, O)


def _e4m3_ties_to_odd(O):
    _set_encode(O, tie_rule="odd")                     # planted: ties to the odd code


def _e4m3_ties_away(O):
    _set_encode(O, tie_rule="away")                    # planted: ties away from zero


def _e4m3_sign_of_zero_lost(O):
    _set_encode(O, keep_zero_sign=False)               # planted: -0 encodes as 0x00


def _scale(floor=True, ceil_rule="mantissa", first_only=False):
    def act_scale_bytes(x_bits, O):
        x = O.bf16_to_f64(x_bits).astype(np.float32)
        K = x.shape[-1]
        if K % O.BLOCK != 0:
            raise O.OracleRefusal("the last dimension is not divisible by 32")
        if not np.all(np.isfinite(x)):
            raise O.OracleRefusal("non-finite activation")
        xb = x.reshape(x.shape[:-1] + (K // O.BLOCK, O.BLOCK))
        amax = np.abs(xb[..., 0]) if first_only else np.abs(xb).max(axis=-1)
        if floor:
            amax = np.maximum(amax, np.float32(1e-4))
        t = (amax * np.float32(1.0 / 448.0)).astype(np.float32)
        bits = t.view(np.uint32)
        bump = ((bits & 0x7FFFFF) != 0) if ceil_rule == "mantissa" else 1
        e = ((bits >> 23) & 0xFF).astype(np.int64) - 127 + bump
        return (e + 127).astype(np.uint8)
    return act_scale_bytes


def _set_scale(O, **kw):
    f = _scale(**kw)
    O.act_scale_bytes = lambda x_bits: f(x_bits, O)


def _scale_no_floor(O):
    _set_scale(O, floor=False)                         # planted: amax not floored at 1e-4


def _scale_always_ceil(O):
    _set_scale(O, ceil_rule="always")                  # planted: +1 even for powers of two


def _scale_first_element_amax(O):
    _set_scale(O, first_only=True)                     # planted: amax of the first element only


def _gemm(drop_bias=False, transpose_b=True, abs_b_in_s=True):
    def gemm_ref(a, b, bias=None):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        bt = np.swapaxes(b, -1, -2) if transpose_b else b
        ref = a @ bt
        S = np.abs(a) @ (np.abs(bt) if abs_b_in_s else bt)
        if bias is not None and not drop_bias:
            ref = ref + np.asarray(bias, dtype=np.float64)[..., None, :]
        return ref, S
    return gemm_ref


def _gemm_drops_bias(O):
    O.gemm_ref = _gemm(drop_bias=True)                 # planted: bias dropped


def _gemm_b_not_transposed(O):
    O.gemm_ref = _gemm(transpose_b=False)              # planted: A . B instead of A . B^T


def _gemm_s_signed(O):
    O.gemm_ref = _gemm(abs_b_in_s=False)               # planted: S = |A| . B^T (sign kept)


def _tolerance_loose(O):
    def within_tolerance(out_bits, ref, S):
        out = O.bf16_to_f64(out_bits)
        ok = np.abs(out - ref) <= np.ldexp(np.abs(ref), -6) + np.ldexp(S, -20)   # planted: 2^-6
        return ok & np.isfinite(out)
    O.within_tolerance = within_tolerance


def _bf16_shift_15(O):
    def bf16_to_f64(bits):
        b = np.asarray(bits, dtype=np.uint16)
        with np.errstate(invalid="ignore"):
            return ((b.astype(np.uint32) << 15)).view(np.float32).astype(np.float64)   # planted
    O.bf16_to_f64 = bf16_to_f64


MUTANTS = {
    "fp4_unpack_high_nibble_first": _fp4_unpack_high_nibble_first,
    "fp4_table_typo": _fp4_table_typo,
    "e8m0_bias_126": _e8m0_bias_126,
    "e4m3_bias_8": _e4m3_bias_8,
    "e4m3_subnormal_step": _e4m3_subnormal_step,
    "fp8_block_scale_transposed": _fp8_block_scale_transposed,
    "e4m3_ties_to_odd": _e4m3_ties_to_odd,
    "e4m3_ties_away": _e4m3_ties_away,
    "e4m3_sign_of_zero_lost": _e4m3_sign_of_zero_lost,
    "scale_no_floor": _scale_no_floor,
    "scale_always_ceil": _scale_always_ceil,
    "scale_first_element_amax": _scale_first_element_amax,
    "gemm_drops_bias": _gemm_drops_bias,
    "gemm_b_not_transposed": _gemm_b_not_transposed,
    "gemm_s_signed": _gemm_s_signed,
    "tolerance_loose": _tolerance_loose,
    "bf16_shift_15": _bf16_shift_15,
}


def pytest_configure(config):
    name = os.environ.get("ORACLE_MUTANT", "none")
    if name == "none":
        return
    from oracle import mx_oracle as O
    MUTANTS[name](O)
