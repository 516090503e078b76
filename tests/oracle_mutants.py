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


# ---- O4 .. O8: the bf16 rounding, the quantized outputs, the MXFP4 producer, the epilogues and
# the backward-pass operands

def _bf16_rne(mode="rint", keep_sign=True):
    def f64_to_bf16_rne(x, O):
        x = np.asarray(x, dtype=np.float64)
        if not np.all(np.isfinite(x)):
            raise O.OracleRefusal("non-finite value")
        ax = np.abs(x)
        _, ex = np.frexp(ax)
        e = np.maximum(ex - 1, -126)
        step = np.ldexp(1.0, e - 7)
        r = ax / step
        n = np.rint(r) if mode == "rint" else np.floor(r) if mode == "floor" else np.floor(r + 0.5)
        v = n * step
        if np.any(v >= np.ldexp(1.0, 128)):
            raise O.OracleRefusal("value rounds past the largest bf16")
        f = (np.copysign(v, x) if keep_sign else v).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    return f64_to_bf16_rne


def _set_bf16_rne(O, **kw):
    f = _bf16_rne(**kw)
    O.f64_to_bf16_rne = lambda x: f(x, O)


def _bf16_rne_floor(O):
    _set_bf16_rne(O, mode="floor")                     # planted: truncation


def _bf16_rne_ties_away(O):
    _set_bf16_rne(O, mode="away")                      # planted: ties away from zero


def _bf16_rne_sign_lost(O):
    _set_bf16_rne(O, keep_sign=False)                  # planted: the sign dropped


def _quant_out_bound_without_t(O):
    def quant_output_within(codes, scale_bytes, ref, S, t=None):
        deq = O.act_qdq_f64(codes, scale_bytes)
        ref = np.asarray(ref, dtype=np.float64)
        if t is None:
            t = np.ldexp(np.abs(ref), -7) + np.ldexp(np.asarray(S, dtype=np.float64), -20)
        t = np.asarray(t, dtype=np.float64)
        E = np.repeat(np.asarray(scale_bytes, dtype=np.int64) - 127, O.BLOCK, axis=-1)
        bound = np.ldexp(np.abs(ref) + t, -4) + np.ldexp(1.0, E - 10)   # planted: + t dropped
        return np.abs(deq - ref) <= bound
    O.quant_output_within = quant_output_within


def _e2m1_ties_to_odd(O):
    def e2m1_encode_rne(y):
        y = np.asarray(y, dtype=np.float64)
        if np.any(~np.isfinite(y)) or np.any(np.abs(y) > 6.0):
            raise O.OracleRefusal("e2m1_encode_rne expects finite |y| <= 6")
        grid = O.e2m1_to_f64(np.arange(8, dtype=np.uint8))
        a = np.abs(y)
        hi = np.minimum(np.searchsorted(grid, a, side="left"), len(grid) - 1)
        lo = np.maximum(hi - 1, 0)
        d_lo, d_hi = a - grid[lo], grid[hi] - a
        pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 1))   # planted: ties to odd
        code = np.where(pick_hi, hi, lo).astype(np.uint8)
        code = np.where(a == grid[hi], hi, code).astype(np.uint8)
        return code | np.where(np.signbit(y), 8, 0).astype(np.uint8)
    O.e2m1_encode_rne = e2m1_encode_rne


def _fp4_pack_swapped(O):
    O.fp4_pack = lambda codes: ((np.asarray(codes, np.uint8)[..., 0::2] << 4)   # planted
                                | np.asarray(codes, np.uint8)[..., 1::2]).astype(np.uint8)


def _fp4_scale(maximum=6.0, bias=127, floor=True):
    def act_scale_fp4_bytes(x_bits, O):
        x = O.bf16_to_f64(x_bits).astype(np.float32)
        K = x.shape[-1]
        if K % O.BLOCK:
            raise O.OracleRefusal("the last dimension is not divisible by 32")
        if not np.all(np.isfinite(x)):
            raise O.OracleRefusal("non-finite activation")
        xb = x.reshape(x.shape[:-1] + (K // O.BLOCK, O.BLOCK))
        amax = np.abs(xb).max(axis=-1)
        if floor:
            amax = np.maximum(amax, np.float32(1e-4))
        amax = amax.astype(np.float64)
        _, ex = np.frexp(amax)
        E = (ex - 1 - 2).astype(np.int64)
        for _ in range(3):
            E = E + (amax > maximum * np.ldexp(1.0, E))
        return (E + bias).astype(np.uint8)
    return act_scale_fp4_bytes


def _set_fp4_scale(O, **kw):
    f = _fp4_scale(**kw)
    O.act_scale_fp4_bytes = lambda x_bits: f(x_bits, O)


def _fp4_scale_max_4(O):
    _set_fp4_scale(O, maximum=4.0)                     # planted: largest E2M1 magnitude 4


def _fp4_scale_bias_126(O):
    _set_fp4_scale(O, bias=126)                        # planted: E8M0 bias 126


def _fp4_scale_no_floor(O):
    _set_fp4_scale(O, floor=False)                     # planted: amax not floored


def _gelu(arg_sign=-1.0, half=0.5):
    def gelu_f64(x):
        from scipy.special import erfc
        x = np.asarray(x, dtype=np.float64)
        return half * x * erfc(arg_sign * x / np.sqrt(2.0))
    return gelu_f64


def _gelu_erfc_sign(O):
    O.gelu_f64 = _gelu(arg_sign=1.0)                   # planted: erfc(+x / sqrt 2)


def _gelu_no_half(O):
    O.gelu_f64 = _gelu(half=1.0)                       # planted: the 1/2 dropped


def _residual_dropped(O):
    O.gemm_residual_ref = lambda a, b, bias=None, residual_bits=None: O.gemm_ref(a, b, bias)


def _gelu_bound_without_s(O):
    def gelu_output_bound(g, S):
        g = np.asarray(g, dtype=np.float64)
        return np.ldexp(np.abs(g), -7) + 2.0 ** -126   # planted: the 2^-19 S term dropped
    O.gelu_output_bound = gelu_output_bound


def _e5m2_bias_16(O):
    def e5m2_to_f64(codes):
        c = np.asarray(codes, dtype=np.uint8)
        if np.any(np.isin(c, O.E5M2_SPECIAL)):
            raise O.OracleRefusal("E5M2 Inf/NaN code")
        s = (c >> 7).astype(np.int64)
        e = ((c >> 2) & 0x1F).astype(np.int64)
        m = (c & 3).astype(np.float64)
        mag = np.where(e == 0, m * 2.0 ** -17, np.ldexp(1.0 + m / 4.0, e - 16))   # planted
        return np.where(s == 1, -mag, mag)
    O.e5m2_to_f64 = e5m2_to_f64


def _philox(rounds=10):
    def philox4x64_10(ctr, key, O):
        with np.errstate(over="ignore"):
            x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in ctr)
            k0, k1 = np.uint64(key[0]), np.uint64(key[1])
            for r in range(rounds):
                if r:
                    k0 = np.uint64((int(k0) + O.PHILOX_W0) & 0xFFFFFFFFFFFFFFFF)
                    k1 = np.uint64((int(k1) + O.PHILOX_W1) & 0xFFFFFFFFFFFFFFFF)
                h0, l0 = O._mulhilo64(x0, O.PHILOX_M0)
                h1, l1 = O._mulhilo64(x2, O.PHILOX_M1)
                x0, x1, x2, x3 = h1 ^ x1 ^ k0, l1, h0 ^ x3 ^ k1, l0
        return x0, x1, x2, x3
    return philox4x64_10


def _philox_9_rounds(O):
    f = _philox(rounds=9)                              # planted: 9 rounds
    O.philox4x64_10 = lambda ctr, key: f(ctr, key, O)


def _philox_multiplier_typo(O):
    O.PHILOX_M1 = O.PHILOX_M1 ^ 0x10                   # planted: one bit of a multiplier


def _uniform_high_half_first(O):
    def uniform_u32(seed, idx):
        idx = np.asarray(idx, dtype=np.uint64)
        blocks, which = np.unique(idx >> np.uint64(3), return_inverse=True)
        z = np.zeros_like(blocks)
        w = O.philox4x64_10((blocks, z, z, z), (np.uint64(seed), np.uint64(0)))
        k = (idx & np.uint64(7)).astype(np.int64).reshape(-1)
        which = which.reshape(-1)
        word = np.choose(k >> 1, [wi[which] for wi in w]).reshape(idx.shape)
        k = k.reshape(idx.shape)
        shift = np.uint64(32) * (1 - (k & 1)).astype(np.uint64)   # planted: high half first
        return ((word >> shift) & np.uint64(0xFFFFFFFF)).astype(np.uint64)
    O.uniform_u32 = uniform_u32


def _stochastic_le(O):
    def e5m2_encode_stochastic(y, u):
        y = np.asarray(y, dtype=np.float64)
        if np.any(~np.isfinite(y)) or np.any(np.abs(y) > 57344.0):
            raise O.OracleRefusal("expects finite |y| <= 57344")
        u = np.asarray(u, dtype=np.uint64).astype(np.float64)
        grid = O.e5m2_to_f64(np.arange(0x7C, dtype=np.uint8))
        a = np.abs(y)
        lo = np.searchsorted(grid, a, side="right") - 1
        on = grid[lo] == a
        hi = np.minimum(lo + 1, len(grid) - 1)
        width = np.where(on, 1.0, grid[hi] - grid[lo])
        up = ~on & (u <= np.ldexp((a - grid[lo]) / width, 32))   # planted: <= for <
        code = np.where(up, hi, lo).astype(np.uint8)
        return code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    O.e5m2_encode_stochastic = e5m2_encode_stochastic


def _grad_scale_no_clamp(O):
    def grad_scale_bytes(x_bits):
        x = O.bf16_to_f64(x_bits).astype(np.float32)
        K = x.shape[-1]
        if K % O.BLOCK:
            raise O.OracleRefusal("the last dimension is not divisible by 32")
        if not np.all(np.isfinite(x)):
            raise O.OracleRefusal("non-finite value")
        xb = x.reshape(x.shape[:-1] + (K // O.BLOCK, O.BLOCK))
        amax = np.maximum(np.abs(xb).max(axis=-1), np.float32(2.0 ** -126)).astype(np.float64)
        _, ex = np.frexp(amax)
        E = (ex - 1 - 15).astype(np.int64)
        for _ in range(2):
            E = E + (amax > 57344.0 * np.ldexp(1.0, E))
        return (E + 127).astype(np.uint8)              # planted: no clamp at -127
    O.grad_scale_bytes = grad_scale_bytes


def _transpose_forgotten(O):
    O.quant_transpose_e4m3 = lambda x_bits: O.act_quant(np.asarray(x_bits))   # planted


def _fp4_out_bound_eighth(O):
    def quant_fp4_output_within(packed, scale_bytes, ref, t):
        deq = O.decode_packed_fp4(packed, scale_bytes)
        ref = np.asarray(ref, dtype=np.float64)
        t = np.asarray(t, dtype=np.float64)
        E = np.repeat(np.asarray(scale_bytes, dtype=np.int64) - 127, O.BLOCK, axis=-1)
        bound = np.ldexp(np.abs(ref) + t, -3) + t + np.ldexp(1.0, E - 2)   # planted: 2^-3
        return np.abs(deq - ref) <= bound
    O.quant_fp4_output_within = quant_fp4_output_within


# name -> (the planting function, the group of pin files that must catch it)
MUTANTS = {
    "fp4_unpack_high_nibble_first": (_fp4_unpack_high_nibble_first, "core"),
    "fp4_table_typo": (_fp4_table_typo, "core"),
    "e8m0_bias_126": (_e8m0_bias_126, "core"),
    "e4m3_bias_8": (_e4m3_bias_8, "core"),
    "e4m3_subnormal_step": (_e4m3_subnormal_step, "core"),
    "fp8_block_scale_transposed": (_fp8_block_scale_transposed, "core"),
    "e4m3_ties_to_odd": (_e4m3_ties_to_odd, "core"),
    "e4m3_ties_away": (_e4m3_ties_away, "core"),
    "e4m3_sign_of_zero_lost": (_e4m3_sign_of_zero_lost, "core"),
    "scale_no_floor": (_scale_no_floor, "core"),
    "scale_always_ceil": (_scale_always_ceil, "core"),
    "scale_first_element_amax": (_scale_first_element_amax, "core"),
    "gemm_drops_bias": (_gemm_drops_bias, "core"),
    "gemm_b_not_transposed": (_gemm_b_not_transposed, "core"),
    "gemm_s_signed": (_gemm_s_signed, "core"),
    "tolerance_loose": (_tolerance_loose, "core"),
    "bf16_shift_15": (_bf16_shift_15, "core"),
    "bf16_rne_floor": (_bf16_rne_floor, "next"),
    "bf16_rne_ties_away": (_bf16_rne_ties_away, "next"),
    "bf16_rne_sign_lost": (_bf16_rne_sign_lost, "next"),
    "quant_out_bound_without_t": (_quant_out_bound_without_t, "next"),
    "e2m1_ties_to_odd": (_e2m1_ties_to_odd, "next"),
    "fp4_pack_swapped": (_fp4_pack_swapped, "next"),
    "fp4_scale_max_4": (_fp4_scale_max_4, "next"),
    "fp4_scale_bias_126": (_fp4_scale_bias_126, "next"),
    "fp4_scale_no_floor": (_fp4_scale_no_floor, "next"),
    "gelu_erfc_sign": (_gelu_erfc_sign, "next"),
    "gelu_no_half": (_gelu_no_half, "next"),
    "residual_dropped": (_residual_dropped, "next"),
    "gelu_bound_without_s": (_gelu_bound_without_s, "next"),
    "e5m2_bias_16": (_e5m2_bias_16, "next"),
    "philox_9_rounds": (_philox_9_rounds, "next"),
    "philox_multiplier_typo": (_philox_multiplier_typo, "next"),
    "uniform_high_half_first": (_uniform_high_half_first, "next"),
    "stochastic_le": (_stochastic_le, "next"),
    "grad_scale_no_clamp": (_grad_scale_no_clamp, "next"),
    "transpose_forgotten": (_transpose_forgotten, "next"),
    "fp4_out_bound_eighth": (_fp4_out_bound_eighth, "next"),
}


def pytest_configure(config):
    name = os.environ.get("ORACLE_MUTANT", "none")
    if name == "none":
        return
    from oracle import mx_oracle as O
    MUTANTS[name][0](O)
