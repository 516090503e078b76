"""Plain CPU oracle for per-32 microscaled activation quantization and the block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and it shares no code, tables or helpers with that path.

Everything here is written to be read against the pages it follows, not to be fast:

* "formats.py" page (the dspark native formats module): module docstring (format contract),
  FP4_TABLE and constants, e8m0_exponents / e8m0_to_f32, fp4_codes / decode_fp4,
  e4m3_codes_to_f32 / decode_fp8_block, _log2_ceil_pow2, act_scale, act_quant, act_qdq, exact_in.
* "hip_quant PKG-INFO" page: "FP8 Formats" table (E4M3 = 1 sign, 4 exponent, 3 mantissa bits,
  bias 7, max 448, NaN only, round to nearest even) and the BF16 checkpoint helper section
  (bf16 -> fp32 is exact from the raw bits).
* "AstrAI commit log" page: the fused-bias commit (the bias joins the fp32 sum, and the GEMM
  output is rounded to bf16 once).
* "fp4-gemm README" page: the epilogue that emits the next projection's quantized input (O4: the
  bf16 GEMM output quantized with act_quant), the MXFP4 operand produced from activations (O5)
  and the bias + residual and bias + GELU epilogues (O6).

Decoded values and the GEMM are carried in float64: every decoded value has at most 4
significant bits times a power of two, so every product of two of them is exact in float64, and
the float64 sum of K such products is within K * 2^-53 * sum|a*b| of the exact sum.

Readings taken where the pages are silent (each is listed in the design notes as well):
* The activation floor 1e-4 is the float32 value nearest 1e-4 (the page clamps a float32 tensor).
* The E8M0 scale output is the byte E + 127 of s = 2^E (the page returns s as float32).
* A negative value that rounds to zero encodes as 0x80 (negative zero), as the float8_e4m3fn
  cast the page uses does.
* The GEMM reference is the unrounded float64 value  sum_k a*b + bias ; the bf16 output is
  accepted when |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a*b|.
* Non-finite activations, NaN E4M3 codes (0x7F, 0xFF) and the NaN scale byte 255 are refused.
* The MXFP4 producer uses act_quant's rule with E2M1's largest magnitude 6 (O5).
* The residual is added before the one rounding to bf16, like the bias; GELU is the exact
  x * Phi(x) of (sum + bias) (O6).

No function here is "parity unpinned" except the GEMM below the stated tolerance (the bf16 output
of any correct implementation may differ from another's inside that bound); the quantized GEMM
output inherits that freedom and is accepted by the bound quant_output_within derives.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32                      # one scale per 32 consecutive values ("formats.py": BLOCK)
FP8_MAX = 448.0                 # largest finite E4M3 magnitude ("formats.py": FP8_MAX)
E8M0_NAN = 255                  # the E8M0 NaN byte ("formats.py": E8M0_NAN)
E4M3_NAN = (0x7F, 0xFF)         # the two e4m3fn NaN bytes ("formats.py": E4M3_NAN)

# E2M1 code -> value, as printed in "formats.py" (FP4_TABLE): sign is bit 3, code 8 is -0.0.
FP4_TABLE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
             -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0)


class OracleRefusal(ValueError):
    """Raised where the pages refuse an input (NaN code, NaN scale, bad shape, non-finite x)."""


# ----------------------------------------------------------------------------------------------
# O1: exact decoders
# ----------------------------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) -> float64.

    "hip_quant PKG-INFO", BF16 checkpoint helper: a bf16 pattern is the top 16 bits of the fp32
    pattern, so widening is exact: fp32 bits = bf16 bits << 16.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e8m0_to_f64(scale_bytes) -> np.ndarray:
    """E8M0 byte b -> 2^(b - 127); byte 255 (NaN) is refused.

    "formats.py": module docstring (E8M0 scale) and e8m0_exponents / e8m0_to_f32.
    """
    s = np.asarray(scale_bytes, dtype=np.uint8)
    n_nan = int(np.count_nonzero(s == E8M0_NAN))
    if n_nan:
        raise OracleRefusal(f"{n_nan} scale byte(s) equal 255, which E8M0 reserves for NaN")
    return np.ldexp(1.0, s.astype(np.int64) - 127)


def fp4_unpack(packed) -> np.ndarray:
    """Packed E2M1 bytes [..., K/2] -> codes [..., K]; byte j holds element 2j in its LOW nibble
    and element 2j+1 in its HIGH nibble.

    "formats.py": module docstring (MXFP4 layout) and fp4_codes.
    """
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    codes[..., 0::2] = p & 0x0F
    codes[..., 1::2] = p >> 4
    return codes


def e2m1_to_f64(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64 through the printed table ("formats.py": FP4_TABLE)."""
    c = np.asarray(codes, dtype=np.uint8)
    if np.any(c > 15):
        raise OracleRefusal("E2M1 code above 15")
    return np.asarray(FP4_TABLE, dtype=np.float64)[c]


def e4m3_to_f64(codes) -> np.ndarray:
    """e4m3fn byte -> float64 from its fields; 0x7F and 0xFF (NaN) are refused.

    "hip_quant PKG-INFO", FP8 Formats table: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits, no infinities.  Exponent field 0 is subnormal: m * 2^-9 (= m/8 * 2^(1-7)).
    Otherwise (1 + m/8) * 2^(e - 7).  "formats.py": e4m3_codes_to_f32 refuses the NaN bytes.
    """
    b = np.asarray(codes, dtype=np.uint8)
    if np.any((b == E4M3_NAN[0]) | (b == E4M3_NAN[1])):
        raise OracleRefusal("E4M3 operand holds NaN codes (0x7F / 0xFF)")
    sign = np.where(b >> 7, -1.0, 1.0)
    e = ((b >> 3) & 0xF).astype(np.int64)
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    return sign * mag


def decode_fp4_rows(packed, scale_bytes) -> np.ndarray:
    """MXFP4 operand [R, K/2] + E8M0 scales [R, K/32] -> float64 [R, K].

    "formats.py": decode_fp4 -- value = FP4_TABLE[code] * 2^(scale - 127), one scale per 32
    consecutive K of one row; K must be a multiple of 32 and the scale shape must match.
    """
    codes = fp4_unpack(packed)
    R, K = codes.shape
    s = np.asarray(scale_bytes, dtype=np.uint8)
    if K % BLOCK or s.shape != (R, K // BLOCK):
        raise OracleRefusal(f"scales shaped {s.shape} do not give each of the {R} rows of {K} "
                            f"E2M1 values one byte per {BLOCK} values")
    v = e2m1_to_f64(codes).reshape(R, K // BLOCK, BLOCK)
    return (v * e8m0_to_f64(s)[:, :, None]).reshape(R, K)


def decode_e4m3_rows(codes, scale_bytes) -> np.ndarray:
    """E4M3 activation codes [R, K] + E8M0 scales [R, K/32] (one per 32 K of a row) -> float64.

    This is the value act_qdq stores: q * s ("formats.py": act_qdq).
    """
    c = np.asarray(codes, dtype=np.uint8)
    R, K = c.shape
    s = np.asarray(scale_bytes, dtype=np.uint8)
    if K % BLOCK or s.shape != (R, K // BLOCK):
        raise OracleRefusal(f"scales shaped {s.shape} do not give each row of the {c.shape} "
                            f"E4M3 codes one byte per {BLOCK} values")
    v = e4m3_to_f64(c).reshape(R, K // BLOCK, BLOCK)
    return (v * e8m0_to_f64(s)[:, :, None]).reshape(R, K)


def decode_fp8_block(codes, scale_bytes) -> np.ndarray:
    """E4M3 weight [N, K] + E8M0 block scales [ceil(N/32), ceil(K/32)] -> float64 [N, K].

    "formats.py": decode_fp8_block -- one scale per 32x32 block; element (n, k) uses scale
    [n // 32, k // 32].
    """
    c = np.asarray(codes, dtype=np.uint8)
    N, K = c.shape
    s = np.asarray(scale_bytes, dtype=np.uint8)
    nb, kb = -(-N // BLOCK), -(-K // BLOCK)
    if s.shape != (nb, kb):
        raise OracleRefusal(f"block scales shaped {s.shape} do not cover the {c.shape} E4M3 "
                            f"weight in {BLOCK}x{BLOCK} blocks")
    scale = e8m0_to_f64(s)
    rows = np.arange(N) // BLOCK
    cols = np.arange(K) // BLOCK
    return e4m3_to_f64(c) * scale[rows[:, None], cols[None, :]]


# ----------------------------------------------------------------------------------------------
# O2: act_quant
# ----------------------------------------------------------------------------------------------

def _e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite e4m3fn values, indexed by their code 0x00..0x7E (increasing)."""
    return e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode_rne(y) -> np.ndarray:
    """Nearest e4m3fn code to each float64 y in [-448, 448], ties to the even code.

    By definition of round-to-nearest-even ("hip_quant PKG-INFO", FP8 Formats: OCP semantics,
    round to nearest even): take the representable magnitude closest to |y|; on a tie take the
    one whose code has an even last mantissa bit.  The magnitudes are the 127 codes 0x00..0x7E in
    increasing order, so the two candidates are found by a sorted search.  The sign bit is the
    sign of y, zero included (-0 -> 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > FP8_MAX):
        raise OracleRefusal("e4m3_encode_rne expects finite |y| <= 448")
    grid = _e4m3_grid()
    a = np.abs(y)
    hi = np.searchsorted(grid, a, side="left")          # grid[hi-1] < a <= grid[hi]
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == grid[hi], hi, code).astype(np.uint8)   # exact hits
    return code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)


def act_scale_bytes(x_bits) -> np.ndarray:
    """Per-32 E8M0 scale bytes of bf16 activations [..., K] -> uint8 [..., K/32].

    "formats.py": act_scale and _log2_ceil_pow2, step by step, in float32 as the page computes:
      amax = max over the 32 of |x| (float32), floored at float32(1e-4);
      t = float32(amax * float32(1/448))  (one float32 multiply, round to nearest even);
      E = exponent field of t - 127, plus 1 when t's mantissa field is non-zero (ceil of log2 t);
      the byte is E + 127.
    K must be a multiple of 32; non-finite activations are refused.
    """
    x = bf16_to_f64(x_bits).astype(np.float32)   # exact: bf16 values are float32 values
    *lead, K = x.shape
    if K % BLOCK != 0:
        raise OracleRefusal(f"act_quant: the last dimension {K} is not divisible by {BLOCK}")
    if not np.all(np.isfinite(x)):
        raise OracleRefusal("act_quant: non-finite activation")
    xb = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.maximum(np.abs(xb).max(axis=-1), np.float32(1e-4))
    t = (amax * np.float32(1.0 / FP8_MAX)).astype(np.float32)
    bits = t.view(np.uint32)
    e = ((bits >> 23) & 0xFF).astype(np.int64) - 127 + ((bits & 0x7FFFFF) != 0)
    return (e + 127).astype(np.uint8)


def act_quant(x_bits) -> tuple[np.ndarray, np.ndarray]:
    """bf16 activations [..., K] -> (E4M3 codes uint8 [..., K], E8M0 scale bytes uint8 [..., K/32]).

    "formats.py": act_quant -- q = e4m3(clamp(x / s, -448, 448)) with round to nearest even.
    x / s is exact in float64 (s is a power of two), the clamp keeps |y| <= 448, and the encode
    is e4m3_encode_rne.
    """
    x = bf16_to_f64(x_bits)
    sb = act_scale_bytes(x_bits)
    K = x.shape[-1]
    s = e8m0_to_f64(sb)
    y = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK)) / s[..., None]
    y = np.clip(y, -FP8_MAX, FP8_MAX)
    codes = e4m3_encode_rne(y).reshape(x.shape)
    return codes, sb


def act_qdq_f64(codes, scale_bytes) -> np.ndarray:
    """q * s as float64 for codes [..., K] and scales [..., K/32] ("formats.py": act_qdq)."""
    c = np.asarray(codes, dtype=np.uint8)
    K = c.shape[-1]
    q = e4m3_to_f64(c).reshape(c.shape[:-1] + (K // BLOCK, BLOCK))
    return (q * e8m0_to_f64(scale_bytes)[..., None]).reshape(c.shape)


def exact_in_bf16(v) -> bool:
    """Every float64 value of v is a finite bf16 value ("formats.py": exact_in, for bf16).

    A finite float64 is a bf16 value when it survives float64 -> float32 unchanged and its
    float32 pattern has zero low 16 bits.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > float(np.finfo(np.float32).max)):
        return False
    f = v.astype(np.float32)
    if not np.all(np.isfinite(f)) or not np.array_equal(f.astype(np.float64), v):
        return False
    return bool(np.all((f.view(np.uint32) & 0xFFFF) == 0))


# ----------------------------------------------------------------------------------------------
# O3: GEMM over exactly decoded operands
# ----------------------------------------------------------------------------------------------

def gemm_ref(a, b, bias=None) -> tuple[np.ndarray, np.ndarray]:
    """(ref, S) for C = A . B^T (+ bias): A [..., M, K], B [..., N, K] float64, bias [..., N].

    ref[m, n] = sum_k A[m,k] B[n,k] + bias[n]   and   S[m, n] = sum_k |A[m,k] B[n,k]|.
    The layout (both operands K-major, output = A times B transposed) is the one the
    "hip_quant PKG-INFO" page states for its FP8 GEMM and its native MXFP4 call.  The bias is
    added to the unrounded sum ("AstrAI commit log": bias in fp32 before the one bf16 rounding;
    here the unrounded float64 value).  The contraction uses the library matmul in float64.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    bt = np.swapaxes(b, -1, -2)
    ref = a @ bt
    S = np.abs(a) @ np.abs(bt)
    if bias is not None:
        ref = ref + np.asarray(bias, dtype=np.float64)[..., None, :]
    return ref, S


def gemm_ref_at(a, b, rows, cols, bias=None) -> tuple[np.ndarray, np.ndarray]:
    """(ref, S) of selected outputs (rows[i], cols[i]) only: one dot product each.

    a [M, K], b [N, K] float64 (one batch).  Used to check full-size outputs by sampling.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    prod = a[rows, :] * b[cols, :]
    ref = prod.sum(axis=1)
    S = np.abs(prod).sum(axis=1)
    if bias is not None:
        ref = ref + np.asarray(bias, dtype=np.float64)[cols]
    return ref, S


def within_tolerance(out_bits, ref, S) -> np.ndarray:
    """Elementwise acceptance of bf16 outputs: |out - ref| <= 2^-7 |ref| + 2^-20 S.

    out_bits are raw bf16 patterns; a NaN or infinite output is never accepted.
    """
    out = bf16_to_f64(out_bits)
    ref = np.asarray(ref, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    ok = np.abs(out - ref) <= np.ldexp(np.abs(ref), -7) + np.ldexp(S, -20)
    return ok & np.isfinite(out)



# ----------------------------------------------------------------------------------------------
# O4: the GEMM output quantized for the next layer (act_quant of the bf16 output)
# ----------------------------------------------------------------------------------------------

def f64_to_bf16_rne(x) -> np.ndarray:
    """float64 -> raw bits (uint16) of the nearest bf16 value, ties to the even significand.

    From the definition of the format: in the binade of |x| (exponent e = floor(log2|x|), and
    e = -126 for the subnormal range) bf16 values are spaced 2^(e-7) apart; |x| is rounded to the
    nearest multiple of that spacing, ties to the even multiple (numpy's rint), and the sign is
    kept (a negative value that rounds to zero gives -0).  The single rounding the GEMM's
    "one bf16 rounding" asks for ("AstrAI commit log": fused-bias commit) applied to the exact
    value.  Non-finite input and values that round past the largest bf16 are refused.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise OracleRefusal("non-finite value")
    ax = np.abs(x)
    _, ex = np.frexp(ax)                       # ax = m * 2^ex with m in [0.5, 1): e = ex - 1
    e = np.maximum(ex - 1, -126)
    step = np.ldexp(1.0, e - 7)
    v = np.rint(ax / step) * step              # both steps exact: power-of-two scalings
    if np.any(v >= np.ldexp(1.0, 128)):
        raise OracleRefusal("value rounds past the largest bf16")
    f = np.copysign(v, x).astype(np.float32)   # exact: v is a bf16 value
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def gemm_act_quant_ref(a, b, bias=None):
    """The GEMM whose output is the next layer's activation operand.

    Returns (ref, S, y_bits, codes, scale_bytes): ref and S as gemm_ref; y_bits = the bf16
    rounding of ref; (codes, scale_bytes) = act_quant(y_bits) per 32 consecutive outputs of a
    row (the "fp4-gemm README" page's quantizing epilogue idea with this library's activation
    format).  Any correct GPU bf16 output may differ from y_bits inside the GEMM tolerance, so
    codes and scale_bytes are exact only for this reference's own rounding; see
    quant_output_within for the acceptance of a GPU result.
    """
    ref, S = gemm_ref(a, b, bias)
    y = f64_to_bf16_rne(ref)
    codes, scales = act_quant(y)
    return ref, S, y, codes, scales


def quant_output_within(codes, scale_bytes, ref, S, t=None) -> np.ndarray:
    """Elementwise acceptance of a quantized GEMM output against the exact ref.

    The GPU's bf16 value y satisfies |y - ref| <= t: by default the GEMM bound
    t = 2^-7 |ref| + 2^-20 S; with GELU before the rounding, the caller passes gelu_within's bound
    (ref then being GELU of the exact sum).  act_quant then rounds y / 2^E to E4M3 with no clamping (the scale rule keeps |y| / 2^E <=
    448): a normal E4M3 value is off by at most half its spacing, 2^-4 of its magnitude, and a
    subnormal one by at most 2^-10, so |q 2^E - y| <= 2^-4 |y| + 2^(E-10).  Together:
        |q 2^E - ref| <= 2^-4 (|ref| + t) + t + 2^(E-10).
    """
    deq = act_qdq_f64(codes, scale_bytes)
    ref = np.asarray(ref, dtype=np.float64)
    if t is None:
        t = np.ldexp(np.abs(ref), -7) + np.ldexp(np.asarray(S, dtype=np.float64), -20)
    t = np.asarray(t, dtype=np.float64)
    E = np.repeat(np.asarray(scale_bytes, dtype=np.int64) - 127, BLOCK, axis=-1)
    bound = np.ldexp(np.abs(ref) + t, -4) + t + np.ldexp(1.0, E - 10)
    return np.abs(deq - ref) <= bound


# ----------------------------------------------------------------------------------------------
# O5: MXFP4 activation producer (bf16 -> packed E2M1 + per-32 E8M0)
# ----------------------------------------------------------------------------------------------
# The pages give the MXFP4 operand format (the formats.py page's FP4_TABLE, nibble order and
# per-32 E8M0 scales; the hip_quant page's native MXFP4 section) but no rule for producing it
# from activations.  The rule used here is act_quant's, with E2M1's largest magnitude 6 in
# place of E4M3's 448 (a reading, listed with the others):
#   amax = max(max |x|, float32(1e-4)) per 32 consecutive values of a row;
#   E = ceil(log2(amax / 6)), exactly: the smallest integer with amax <= 6 * 2^E, so every x / 2^E
#       lies in [-6, 6] and nothing is clipped;
#   code = the E2M1 value nearest x / 2^E (exact: a power-of-two scaling), ties to the even code,
#       the sign kept (a negative value that rounds to zero is code 8);
#   byte = E + 127; codes packed two per byte, element 2j in the low nibble of byte j.

FP4_MAX = 6.0


def e2m1_encode_rne(y) -> np.ndarray:
    """Nearest E2M1 code to each float64 y in [-6, 6], ties to the even code, sign kept.

    The 8 magnitudes are the printed table's codes 0..7 in increasing order ("formats.py":
    FP4_TABLE); the two candidates around |y| are found by a sorted search, as for E4M3.
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > FP4_MAX):
        raise OracleRefusal("e2m1_encode_rne expects finite |y| <= 6")
    grid = e2m1_to_f64(np.arange(8, dtype=np.uint8))
    a = np.abs(y)
    hi = np.minimum(np.searchsorted(grid, a, side="left"), len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == grid[hi], hi, code).astype(np.uint8)
    return code | np.where(np.signbit(y), 8, 0).astype(np.uint8)


def fp4_pack(codes) -> np.ndarray:
    """E2M1 codes [..., K] -> packed bytes [..., K/2]: element 2j low nibble, 2j+1 high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def act_scale_fp4_bytes(x_bits) -> np.ndarray:
    """Per-32 E8M0 bytes of the MXFP4 producer: E + 127 with E = ceil(log2(amax / 6)) exactly.

    amax is taken in float32 as act_scale does (bf16 values are float32 values; the floor is
    float32(1e-4)).  E starts from floor(log2 amax) - 2 (frexp, exact) and is raised while
    amax > 6 * 2^E (exact float64 comparisons).
    """
    x = bf16_to_f64(x_bits).astype(np.float32)
    K = x.shape[-1]
    if K % BLOCK:
        raise OracleRefusal(f"act_quant_fp4: the last dimension {K} is not divisible by {BLOCK}")
    if not np.all(np.isfinite(x)):
        raise OracleRefusal("act_quant_fp4: non-finite activation")
    xb = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.maximum(np.abs(xb).max(axis=-1), np.float32(1e-4)).astype(np.float64)
    _, ex = np.frexp(amax)
    E = (ex - 1 - 2).astype(np.int64)
    for _ in range(3):
        E = E + (amax > FP4_MAX * np.ldexp(1.0, E))
    return (E + 127).astype(np.uint8)


def act_quant_fp4(x_bits) -> tuple[np.ndarray, np.ndarray]:
    """bf16 activations [..., K] -> (packed E2M1 uint8 [..., K/2], E8M0 bytes uint8 [..., K/32])."""
    x = bf16_to_f64(x_bits)
    sb = act_scale_fp4_bytes(x_bits)
    K = x.shape[-1]
    y = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK)) / e8m0_to_f64(sb)[..., None]
    codes = e2m1_encode_rne(y).reshape(x.shape)
    return fp4_pack(codes), sb


# ----------------------------------------------------------------------------------------------
# O6: residual and GELU epilogues
# ----------------------------------------------------------------------------------------------
# The "fp4-gemm README" page lists GEMM epilogues that add a residual (bias + residual, and
# residual alone) or apply GELU after the bias, so that the output feeds the next low-bit GEMM
# without a separate elementwise pass; it gives no formula for either.  Readings used here (each
# is listed with the others):
#   residual: out = one bf16 rounding of (sum_k a*b + bias[n] + residual[m, n]); the residual is
#       a bf16 [M, N] tensor added before the single rounding, like the bias;
#   GELU: the exact form x * Phi(x), Phi the standard normal CDF, applied to (sum_k a*b + bias[n])
#       before the single rounding.

GELU_LIPSCHITZ = 1.128905                # >= max |d/dx x Phi(x)| = Phi(sqrt 2) + sqrt 2 phi(sqrt 2)


def gelu_f64(x) -> np.ndarray:
    """x * Phi(x) in float64, written as 0.5 x erfc(-x / sqrt 2).

    erfc (the library routine) rather than 1 + erf keeps the relative accuracy where Phi(x) is
    tiny (large negative x), where 1 + erf(x / sqrt 2) would cancel.
    """
    from scipy.special import erfc
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * erfc(-x / np.sqrt(2.0))


def gemm_residual_ref(a, b, bias=None, residual_bits=None) -> tuple[np.ndarray, np.ndarray]:
    """(ref, S): gemm_ref with the bf16 residual [..., M, N] added to the unrounded value.

    The residual enters like the bias, before the one rounding to bf16, so the GEMM acceptance
    bound applies unchanged to out against this ref.
    """
    ref, S = gemm_ref(a, b, bias)
    if residual_bits is not None:
        ref = ref + bf16_to_f64(residual_bits)
    return ref, S


def gemm_gelu_ref(a, b, bias=None) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(g, pre, S): g = gelu_f64(pre), pre = sum_k a*b + bias (gemm_ref), S = sum_k |a*b|."""
    pre, S = gemm_ref(a, b, bias)
    return gelu_f64(pre), pre, S


def gelu_within(out_bits, pre, S) -> np.ndarray:
    """Elementwise acceptance of a bf16 GELU output against the exact pre-activation value pre.

    The GPU accumulator a meets the GEMM's accuracy, |a - pre| <= 2^-20 S; GELU is Lipschitz with
    constant GELU_LIPSCHITZ < 2, so |gelu(a) - gelu(pre)| <= 2^-19 S; the float32 evaluation of
    GELU and the one bf16 rounding add at most 2^-7 |gelu(pre)| (bf16 alone is 2^-9); values in
    the bf16 subnormal range are resolved to 2^-126 at best.  Accepted when
        |out - gelu(pre)| <= 2^-7 |gelu(pre)| + 2^-19 S + 2^-126.
    A NaN or infinite output is never accepted.
    """
    out = bf16_to_f64(out_bits)
    g = gelu_f64(pre)
    ok = np.abs(out - g) <= gelu_output_bound(g, S)
    return ok & np.isfinite(out)


def gelu_output_bound(g, S) -> np.ndarray:
    """The bound of gelu_within, 2^-7 |g| + 2^-19 S + 2^-126, for g = GELU of the exact sum: what
    a GPU bf16 GELU output is within, and so the t of the quantized-output checks after GELU."""
    g = np.asarray(g, dtype=np.float64)
    return np.ldexp(np.abs(g), -7) + np.ldexp(np.asarray(S, dtype=np.float64), -19) + 2.0 ** -126


# ----------------------------------------------------------------------------------------------
# O7: backward-pass operands: E5M2 gradients (round-to-nearest-even or stochastic) and
#     quantize-transpose
# ----------------------------------------------------------------------------------------------
# The hip_quant page's "FP8 Formats" table gives E5M2 as 1 sign, 5 exponent, 2 mantissa bits,
# bias 15, max 57344, with Inf and NaN; its default rounding is round-to-nearest-even, and its
# opt-in stochastic rounding for backward gradients picks one of the two E5M2 values around the
# input, the nearer one more often in proportion to how near it is, with randomness that depends
# only on a seed and the element's position (a hash, no generator state).  It also offers
# quantize-plus-transpose for rank-2 tensors, and block-wise E5M2 with one scale per 32 values
# along the last dimension; the AstrAI page feeds the weight and input gradients to the forward
# GEMM through transposed copies.  Readings (each
# is listed with the others):
#   scale: act_quant's rule with E5M2's largest magnitude 57344: E = ceil(log2(amax / 57344))
#       exactly, amax floored at the smallest normal float32 (a gradient block may be far
#       below act_quant's 1e-4 floor), E clamped to E8M0's least exponent -127;
#   stochastic rounding: with lo <= |y| < hi the neighbouring E5M2 magnitudes, the result is hi
#       when u < 2^32 (|y| - lo) / (hi - lo), else lo, for a 32-bit uniform u;
#   the hash: Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
#       SC 2011) with key (seed, 0) and counter (i >> 3, 0, 0, 0); the element with index i takes
#       32-bit word i & 7 of the block (64-bit output word (i & 7) >> 1, low half first);
#   the element index is the position of the code in the quantized output (row-major), so a
#       transposed output draws by its own layout.

E5M2_MAX = 57344.0
E5M2_SPECIAL = tuple(range(0x7C, 0x80)) + tuple(range(0xFC, 0x100))    # Inf and NaN codes


def e5m2_to_f64(codes) -> np.ndarray:
    """E5M2 code -> value from its bit fields (hip_quant page, FP8 Formats table): sign bit 7,
    exponent bits 6..2 with bias 15, 2 mantissa bits; exponent 0 is subnormal, m * 2^-16.
    Inf and NaN codes (exponent 31) are refused."""
    c = np.asarray(codes, dtype=np.uint8)
    if np.any(np.isin(c, E5M2_SPECIAL)):
        raise OracleRefusal("E5M2 Inf/NaN code")
    s = (c >> 7).astype(np.int64)
    e = ((c >> 2) & 0x1F).astype(np.int64)
    m = (c & 3).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -16, np.ldexp(1.0 + m / 4.0, e - 15))
    return np.where(s == 1, -mag, mag)


def _e5m2_grid() -> np.ndarray:
    """The 124 non-negative finite E5M2 magnitudes in increasing order (codes 0x00..0x7B)."""
    return e5m2_to_f64(np.arange(0x7C, dtype=np.uint8))


def e5m2_encode_rne(y) -> np.ndarray:
    """Nearest E5M2 code to each float64 y with |y| <= 57344, ties to the even code, sign kept."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E5M2_MAX):
        raise OracleRefusal("e5m2_encode_rne expects finite |y| <= 57344")
    grid = _e5m2_grid()
    a = np.abs(y)
    hi = np.minimum(np.searchsorted(grid, a, side="left"), len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == grid[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)


def grad_scale_bytes(x_bits) -> np.ndarray:
    """Per-32 E8M0 bytes of the gradient quantizer: E + 127, E = ceil(log2(amax / 57344)) exactly,
    amax (float32, from bf16) floored at 2^-126, E clamped to >= -127.  E starts from
    floor(log2 amax) - 15 (frexp, exact) and is raised while amax > 57344 * 2^E."""
    x = bf16_to_f64(x_bits).astype(np.float32)
    K = x.shape[-1]
    if K % BLOCK:
        raise OracleRefusal(f"gradient quantizer: the last dimension {K} is not divisible by {BLOCK}")
    if not np.all(np.isfinite(x)):
        raise OracleRefusal("gradient quantizer: non-finite value")
    xb = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.maximum(np.abs(xb).max(axis=-1), np.float32(2.0 ** -126)).astype(np.float64)
    _, ex = np.frexp(amax)
    E = (ex - 1 - 15).astype(np.int64)
    for _ in range(2):
        E = E + (amax > E5M2_MAX * np.ldexp(1.0, E))
    return (np.maximum(E, -127) + 127).astype(np.uint8)


_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_LO32 = np.uint64(0xFFFFFFFF)
PHILOX_M0, PHILOX_M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157    # round multipliers
PHILOX_W0, PHILOX_W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B    # key increments (Weyl)


def _mulhilo64(a: np.ndarray, m: int):
    """(high, low) 64-bit halves of the 128-bit product a * m, from 32-bit pieces."""
    a = a.astype(np.uint64)
    a0, a1 = a & _LO32, a >> np.uint64(32)
    m0, m1 = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> np.uint64(32)) + (p01 & _LO32) + (p10 & _LO32)
    lo = (mid << np.uint64(32)) | (p00 & _LO32)
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds (Salmon et al., SC 2011): ctr a tuple of 4 uint64 arrays, key a
    tuple of 2 uint64 values; returns the 4 output words.  A round maps (x0, x1, x2, x3) with
    (h0, l0) = M0 * x0 and (h1, l1) = M1 * x2 to (h1 ^ x1 ^ k0, l1, h0 ^ x3 ^ k1, l0); the key
    advances by (W0, W1) between rounds."""
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in ctr)
        k0, k1 = np.uint64(key[0]), np.uint64(key[1])
        for r in range(10):
            if r:
                k0 = np.uint64((int(k0) + PHILOX_W0) & 0xFFFFFFFFFFFFFFFF)
                k1 = np.uint64((int(k1) + PHILOX_W1) & 0xFFFFFFFFFFFFFFFF)
            h0, l0 = _mulhilo64(x0, PHILOX_M0)
            h1, l1 = _mulhilo64(x2, PHILOX_M1)
            x0, x1, x2, x3 = h1 ^ x1 ^ k0, l1, h0 ^ x3 ^ k1, l0
    return x0, x1, x2, x3


def uniform_u32(seed: int, idx) -> np.ndarray:
    """The 32-bit uniform of element index idx: word idx & 7 of Philox4x64-10 block idx >> 3
    under key (seed, 0) (64-bit output word (idx & 7) >> 1, low half first)."""
    idx = np.asarray(idx, dtype=np.uint64)
    blocks, which = np.unique(idx >> np.uint64(3), return_inverse=True)   # each block once
    z = np.zeros_like(blocks)
    w = philox4x64_10((blocks, z, z, z), (np.uint64(seed), np.uint64(0)))
    k = (idx & np.uint64(7)).astype(np.int64).reshape(-1)
    which = which.reshape(-1)
    word = np.choose(k >> 1, [wi[which] for wi in w]).reshape(idx.shape)
    k = k.reshape(idx.shape)
    return ((word >> (np.uint64(32) * (k & 1).astype(np.uint64))) & _LO32).astype(np.uint64)


def e5m2_encode_stochastic(y, u) -> np.ndarray:
    """Stochastic E5M2 code of each float64 y (|y| <= 57344) under 32-bit uniforms u: with
    lo <= |y| < hi the neighbouring E5M2 magnitudes, hi when u < 2^32 (|y| - lo) / (hi - lo),
    else lo (|y| on the grid is kept); the sign of y is kept.  All quantities are dyadic, so the
    comparison is exact in float64."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E5M2_MAX):
        raise OracleRefusal("e5m2_encode_stochastic expects finite |y| <= 57344")
    u = np.asarray(u, dtype=np.uint64).astype(np.float64)           # exact: < 2^53
    grid = _e5m2_grid()
    a = np.abs(y)
    lo = np.searchsorted(grid, a, side="right") - 1                  # grid[lo] <= a
    on = grid[lo] == a
    hi = np.minimum(lo + 1, len(grid) - 1)
    width = np.where(on, 1.0, grid[hi] - grid[lo])
    up = ~on & (u < np.ldexp((a - grid[lo]) / width, 32))
    code = np.where(up, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)


def grad_quant_e5m2(x_bits, seed=None) -> tuple[np.ndarray, np.ndarray]:
    """bf16 gradients [..., K] -> (E5M2 codes [..., K], E8M0 bytes [..., K/32]) per 32 along the
    last dimension: y = x / 2^E (exact), then round-to-nearest-even (seed None) or stochastic
    rounding with u = uniform_u32(seed, i), i the element's row-major index in the output."""
    x = bf16_to_f64(x_bits)
    sb = grad_scale_bytes(x_bits)
    K = x.shape[-1]
    y = (x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK)) / e8m0_to_f64(sb)[..., None]).reshape(x.shape)
    if seed is None:
        codes = e5m2_encode_rne(y)
    else:
        u = uniform_u32(seed, np.arange(y.size, dtype=np.uint64)).reshape(y.shape)
        codes = e5m2_encode_stochastic(y, u)
    return codes, sb


def quant_transpose_e4m3(x_bits) -> tuple[np.ndarray, np.ndarray]:
    """bf16 [R, C] -> act_quant of its transpose: E4M3 codes [C, R] and E8M0 bytes [C, R/32], the
    32-blocks running along R (the contraction dimension of a GEMM that reads the transpose)."""
    x = np.asarray(x_bits)
    if x.ndim != 2:
        raise OracleRefusal("quant_transpose expects a rank-2 tensor")
    return act_quant(np.ascontiguousarray(x.T))


def quant_transpose_e5m2(x_bits, seed=None) -> tuple[np.ndarray, np.ndarray]:
    """bf16 [R, C] -> grad_quant_e5m2 of its transpose (codes [C, R], bytes [C, R/32]); the
    stochastic draw uses each code's index in that [C, R] output."""
    x = np.asarray(x_bits)
    if x.ndim != 2:
        raise OracleRefusal("quant_transpose expects a rank-2 tensor")
    return grad_quant_e5m2(np.ascontiguousarray(x.T), seed)


def decode_e5m2_rows(codes, scale_bytes) -> np.ndarray:
    """E5M2 codes [..., K] with per-row-32 scales [..., K/32] -> float64 values."""
    v = e5m2_to_f64(codes)
    s = np.repeat(e8m0_to_f64(scale_bytes), BLOCK, axis=-1)
    return v * s


# ----------------------------------------------------------------------------------------------
# O8: the GEMM output quantized to MXFP4 for the next A4W4 layer (with or without GELU)
# ----------------------------------------------------------------------------------------------
# The fp4-gemm README page's bias + GELU epilogue emits packed FP4 with its scales, so that the
# next projection reads it directly.  Here the output format is this library's MXFP4 activation
# operand: y = the bf16 GEMM output (O3, or GELU of it, O6), then act_quant_fp4(y) (O5).

def gemm_quant_fp4_ref(a, b, bias=None, gelu=False):
    """(ref, S, y_bits, packed, scale_bytes): ref = sum_k a*b + bias (gelu: GELU of it) in float64,
    S = sum_k |a*b|, y_bits = its bf16 rounding, (packed, scale_bytes) = act_quant_fp4(y_bits)."""
    pre, S = gemm_ref(a, b, bias)
    ref = gelu_f64(pre) if gelu else pre
    y = f64_to_bf16_rne(ref)
    packed, scales = act_quant_fp4(y)
    return ref, S, y, packed, scales


def decode_packed_fp4(packed, scale_bytes) -> np.ndarray:
    """Packed E2M1 [..., N/2] with per-32 E8M0 bytes [..., N/32] -> float64 [..., N]."""
    return decode_fp4_rows(packed, scale_bytes)


def quant_fp4_output_within(packed, scale_bytes, ref, t) -> np.ndarray:
    """Elementwise acceptance of an MXFP4-quantized GEMM output against the exact ref, given the
    bound t that the bf16 value y the GPU quantized meets (|y - ref| <= t: the GEMM bound, or the
    GELU bound).  MXFP4 rounding of y / 2^E (|y| / 2^E <= 6, no clamping) moves a value in [1, 6]
    by at most a quarter of it (spacings 0.5, 1, 2 on [1, 2), [2, 4), [4, 6]) and a value below 1
    by at most 0.25, so |q 2^E - y| <= 2^-2 |y| + 2^(E-2).  Together:
        |q 2^E - ref| <= 2^-2 (|ref| + t) + t + 2^(E-2).
    """
    deq = decode_packed_fp4(packed, scale_bytes)
    ref = np.asarray(ref, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    E = np.repeat(np.asarray(scale_bytes, dtype=np.int64) - 127, BLOCK, axis=-1)
    bound = np.ldexp(np.abs(ref) + t, -2) + t + np.ldexp(1.0, E - 2)
    return np.abs(deq - ref) <= bound
