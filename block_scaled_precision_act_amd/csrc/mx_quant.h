// Per-32 E4M3 + E8M0 quantization of bf16 values held in registers, for gfx950 kernels: the one
// implementation act_quant and the quantizing GEMM epilogue share, so both produce the same bytes
// for the same bf16 input.
//
// Semantics ("formats.py" page: act_scale, _log2_ceil_pow2, act_quant), per 32 consecutive
// elements of a row:
//   amax = max(max |x|, fp32(1e-4)); t = fp32(amax * fp32(1/448));
//   E = exponent field of t - 127, plus one when t's mantissa is non-zero; byte = E + 127;
//   q = e4m3_rne(clamp(x * 2^-E, -448, 448)).
// x * 2^-E is exact (a power-of-two scaling that cannot overflow, and an underflowing product
// rounds to a signed zero, as the exact value does), and v_cvt_pk_fp8_f32 rounds to nearest even
// into OCP e4m3fn with subnormals and signed zero.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mx {

constexpr uint32_t kInv448Bits = 0x3B124925u;   // fp32(1/448)

// quad_perm [1,0,3,2] then [2,3,0,1]: every lane of a DPP quad ends with the quad's max.  All
// four lanes of the quad must be active.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

// Largest |bf16| bit pattern of 8 packed bf16: |bf16| patterns compare as unsigned integers
// exactly like the values they encode.
__device__ __forceinline__ uint32_t abs_max_bits(uint4 w) {
  uint32_t m01 = max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu);
  uint32_t m23 = max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu);
  uint32_t m45 = max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu);
  uint32_t m67 = max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu);
  return max(max(m01, m23), max(m45, m67));
}

__device__ __forceinline__ float clamp448(float y) {
  return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f);
}

// Four bf16 (two packed pairs) times inv_s -> four E4M3 codes in one dword (element order kept).
__device__ __forceinline__ uint32_t encode4(uint32_t lo_pair, uint32_t hi_pair, float inv_s) {
  float y0 = clamp448(__uint_as_float(lo_pair << 16) * inv_s);
  float y1 = clamp448(__uint_as_float(lo_pair & 0xFFFF0000u) * inv_s);
  float y2 = clamp448(__uint_as_float(hi_pair << 16) * inv_s);
  float y3 = clamp448(__uint_as_float(hi_pair & 0xFFFF0000u) * inv_s);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, r, true);
  return static_cast<uint32_t>(r);
}

struct QuantChunk {
  uint2 codes;      // E4M3 codes of the lane's 8 values
  uint32_t byte;    // E8M0 byte of the 32-block (E + 127, in [105, 247])
};

// E8M0 byte of a 32-block from the largest |bf16| pattern of the block.
__device__ __forceinline__ uint32_t act_scale_byte(uint32_t amax_bits) {
  const float amax = fmaxf(__uint_as_float(amax_bits << 16), 1e-4f);
  const uint32_t t = __float_as_uint(amax * __uint_as_float(kInv448Bits));
  return (t >> 23) + ((t & 0x7FFFFFu) != 0u);
}

// The lane holds 8 consecutive bf16 of a row; the four lanes of its DPP quad hold one 32-block.
__device__ __forceinline__ QuantChunk quant_chunk(uint4 w) {
  QuantChunk r;
  r.byte = act_scale_byte(quad_max(abs_max_bits(w)));
  const float inv_s = __uint_as_float((254u - r.byte) << 23);     // 2^-E, a normal fp32
  r.codes.x = encode4(w.x, w.y, inv_s);
  r.codes.y = encode4(w.z, w.w, inv_s);
  return r;
}

}  // namespace mx

namespace mx {

// The MXFP4 producer of the same 32-blocks: E = ceil(log2(amax / 6)) exactly, where
// amax = max(max |x|, fp32(1e-4)) = m * 2^e with m in [1, 2): amax / 6 = (m / 1.5) * 2^(e-2) and
// m / 1.5 lies in [2/3, 4/3), so E = e - 2, plus one when m > 1.5 (mantissa field > 0x400000).
// x / 2^E then lies in [-6, 6]; v_cvt_scalef32_pk_fp4_f32 divides by the scale 2^E (exact) and
// rounds to the nearest E2M1 value, ties to the even code, keeping the sign (checked on the device
// for every bf16 value).  Codes are packed low nibble first: the lane's 8 values give one dword.
struct QuantChunkFp4 {
  uint32_t codes;   // 8 E2M1 codes, element 0 in the low nibble
  uint32_t byte;    // E8M0 byte of the 32-block
};

// E8M0 byte of a 32-block for MXFP4 from the largest |bf16| pattern of the block.
__device__ __forceinline__ uint32_t fp4_scale_byte(uint32_t amax_bits) {
  const uint32_t ab = __float_as_uint(fmaxf(__uint_as_float(amax_bits << 16), 1e-4f));
  return ((ab >> 23) & 0xFFu) - 2u + ((ab & 0x7FFFFFu) > 0x400000u);
}

// Four bf16 (two packed pairs) divided by s = 2^E -> four E2M1 codes in the low 16 bits
// (element 0 in the low nibble).
__device__ __forceinline__ uint32_t encode4_fp4(uint32_t lo_pair, uint32_t hi_pair, float s) {
  uint32_t c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, __uint_as_float(lo_pair << 16),
                                               __uint_as_float(lo_pair & 0xFFFF0000u), s, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, __uint_as_float(hi_pair << 16),
                                               __uint_as_float(hi_pair & 0xFFFF0000u), s, 1);
  return c;
}

__device__ __forceinline__ QuantChunkFp4 quant_chunk_fp4(uint4 w) {
  QuantChunkFp4 r;
  r.byte = fp4_scale_byte(quad_max(abs_max_bits(w)));
  const float s = __uint_as_float(r.byte << 23);                 // 2^E, a normal fp32
  r.codes = encode4_fp4(w.x, w.y, s) | (encode4_fp4(w.z, w.w, s) << 16);
  return r;
}

}  // namespace mx

namespace mx {

// E5M2 gradients (hip_quant page, FP8 Formats table: 1 sign, 5 exponent bits with bias 15,
// 2 mantissa bits, largest magnitude 57344 = 1.75 * 2^15), per 32 consecutive elements with an
// E8M0 scale: E = ceil(log2(amax / 57344)) exactly, amax floored at 2^-126 and E at -127.  With
// amax = m * 2^e (m in [1, 2)), amax <= 1.75 * 2^(15 + E) holds first for E = e - 15 when
// m <= 1.75 (mantissa field <= 0x600000), else for E = e - 14.
__device__ __forceinline__ uint32_t e5m2_scale_byte(uint32_t amax_bf16_bits) {
  const uint32_t ab = max(amax_bf16_bits << 16, 0x00800000u);      // fp32 bits, floor 2^-126
  const int byte = static_cast<int>(ab >> 23) - 15 + ((ab & 0x7FFFFFu) > 0x600000u);
  return static_cast<uint32_t>(max(byte, 0));
}

// Round-to-nearest-even of four bf16 (two packed pairs) times inv_s into four E5M2 codes
// (v_cvt_pk_bf8_f32: OCP E5M2, ties to even, subnormals and signed zero; |x * inv_s| <= 57344).
__device__ __forceinline__ uint32_t encode4_e5m2(uint32_t lo_pair, uint32_t hi_pair, float inv_s) {
  const float y0 = __uint_as_float(lo_pair << 16) * inv_s;
  const float y1 = __uint_as_float(lo_pair & 0xFFFF0000u) * inv_s;
  const float y2 = __uint_as_float(hi_pair << 16) * inv_s;
  const float y3 = __uint_as_float(hi_pair & 0xFFFF0000u) * inv_s;
  int r = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
  r = __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, r, true);
  return static_cast<uint32_t>(r);
}

// Stochastic E5M2 code of y (|y| <= 57344) under the 32-bit uniform u: with lo <= |y| < hi the
// neighbouring E5M2 magnitudes, the code of hi when u < 2^32 (|y| - lo) / (hi - lo), else of lo;
// the sign of y is kept.  Integer-exact: for |y| >= 2^-14 (E5M2 normals) lo keeps the top two
// mantissa bits of |y|, the fraction is the 21 dropped bits over 2^21 and the threshold is those
// bits times 2^11; below, the grid step is 2^-16 and q = |y| * 2^16, its integer part k and
// (q - k) * 2^32 are exact in fp32.  A code plus one is the next E5M2 magnitude up.
__device__ __forceinline__ uint32_t e5m2_sr_code(float y, uint32_t u) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t mag, thr;
  if (a >= 0x38800000u) {
    mag = (((a >> 23) - 112u) << 2) | ((a >> 21) & 3u);
    thr = (a & 0x1FFFFFu) << 11;
  } else {
    const float q = __uint_as_float(a) * 65536.0f;
    const float k = floorf(q);
    mag = static_cast<uint32_t>(k);
    thr = static_cast<uint32_t>(ceilf((q - k) * 4294967296.0f));
  }
  mag += u < thr ? 1u : 0u;
  return ((b >> 24) & 0x80u) | mag;
}

// Four bf16 (two packed pairs) times inv_s, stochastically rounded with u[0..3], into one dword
// of four codes (element order kept).
__device__ __forceinline__ uint32_t encode4_e5m2_sr(uint32_t lo_pair, uint32_t hi_pair,
                                                    float inv_s, uint32_t u0, uint32_t u1,
                                                    uint32_t u2, uint32_t u3) {
  const uint32_t c0 = e5m2_sr_code(__uint_as_float(lo_pair << 16) * inv_s, u0);
  const uint32_t c1 = e5m2_sr_code(__uint_as_float(lo_pair & 0xFFFF0000u) * inv_s, u1);
  const uint32_t c2 = e5m2_sr_code(__uint_as_float(hi_pair << 16) * inv_s, u2);
  const uint32_t c3 = e5m2_sr_code(__uint_as_float(hi_pair & 0xFFFF0000u) * inv_s, u3);
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// 2^-E for an E8M0 byte E + 127 in [0, 253]: a normal fp32.
__device__ __forceinline__ float inv_scale_of_byte(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

}  // namespace mx
