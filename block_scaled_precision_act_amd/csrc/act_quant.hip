// act_quant for gfx950: bf16 [M, K] -> E4M3 codes [M, K] + E8M0 scale bytes [M, K/32].
//
// Semantics ("formats.py" page: act_scale, _log2_ceil_pow2, act_quant), per 32 consecutive
// elements of a row:
//   amax = max(max |x|, fp32(1e-4)); t = fp32(amax * fp32(1/448));
//   E = exponent field of t - 127, plus one when t's mantissa is non-zero; byte = E + 127;
//   q = e4m3_rne(clamp(x * 2^-E, -448, 448)).
//
// Bandwidth design: a row's 32-blocks are contiguous and K % 32 == 0, so a contiguous [M, K]
// matrix is one flat run of 32-blocks and scale byte i belongs to elements [32i, 32i+32).
// Each lane owns one 16-byte chunk (8 bf16) per step; the four lanes of a DPP quad own one
// block, so the block max needs two quad permutes and no LDS.  Loads are 16 B, stores of codes
// are 8 B per lane (512 contiguous bytes per wavefront), the scale byte is written by the
// quad's first lane; code and scale stores are non-temporal (streamed past the caches).
// x * 2^-E is exact (a power-of-two scaling that cannot overflow, and an
// underflowing product rounds to a signed zero, as the exact value does), and
// v_cvt_pk_fp8_f32 rounds to nearest even into OCP e4m3fn with subnormals and signed zero.
#include "mx_internal.h"

namespace mx {
namespace {

constexpr uint32_t kInv448Bits = 0x3B124925u;   // fp32(1/448)
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of the quad ends with the quad's max.
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ uint32_t abs_max_bits(uint4 w) {
  // |bf16| patterns compare as unsigned integers exactly like the values they encode.
  uint32_t m01 = max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu);
  uint32_t m23 = max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu);
  uint32_t m45 = max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu);
  uint32_t m67 = max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu);
  return max(max(m01, m23), max(m45, m67));
}

__device__ __forceinline__ float clamp448(float y) {
  return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f);
}

__device__ __forceinline__ uint32_t encode4(uint32_t lo_pair, uint32_t hi_pair, float inv_s) {
  float y0 = clamp448(__uint_as_float(lo_pair << 16) * inv_s);
  float y1 = clamp448(__uint_as_float(lo_pair & 0xFFFF0000u) * inv_s);
  float y2 = clamp448(__uint_as_float(hi_pair << 16) * inv_s);
  float y3 = clamp448(__uint_as_float(hi_pair & 0xFFFF0000u) * inv_s);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, r, true);
  return static_cast<uint32_t>(r);
}

// grid.x covers ceil(chunks / (kThreads * UNROLL)) slots, grid.y is the batch index.
// UNROLL: 16-byte chunks in flight per lane; NT: non-temporal code and scale stores.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ s,
    int64_t chunks, int64_t stride_x, int64_t stride_q, int64_t stride_s) {
  const int64_t bz = blockIdx.y;
  const uint4* xv = reinterpret_cast<const uint4*>(x + bz * stride_x);
  uint2* qv = reinterpret_cast<uint2*>(q + bz * stride_q);
  uint8_t* sv = s + bz * stride_s;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * UNROLL) + threadIdx.x;

  uint4 w[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t c = base + u * kThreads;
    w[u] = c < chunks ? xv[c] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t c = base + u * kThreads;
    // A quad's four chunks are all in range or all out of range (chunks % 4 == 0 and quads
    // start at multiples of 4), so the quad permute below only mixes live lanes.
    uint32_t amax_bits = quad_max(abs_max_bits(w[u]));
    float amax = fmaxf(__uint_as_float(amax_bits << 16), 1e-4f);
    uint32_t t = __float_as_uint(amax * __uint_as_float(kInv448Bits));
    uint32_t byte = (t >> 23) + ((t & 0x7FFFFFu) != 0u);      // E + 127, in [105, 247]
    float inv_s = __uint_as_float((254u - byte) << 23);       // 2^-E, a normal fp32
    if (c < chunks) {
      uint2 codes;
      codes.x = encode4(w[u].x, w[u].y, inv_s);
      codes.y = encode4(w[u].z, w[u].w, inv_s);
      if (NT) {
        __builtin_nontemporal_store(codes.x, reinterpret_cast<uint32_t*>(qv + c));
        __builtin_nontemporal_store(codes.y, reinterpret_cast<uint32_t*>(qv + c) + 1);
        if ((threadIdx.x & 3) == 0) __builtin_nontemporal_store(static_cast<uint8_t>(byte), sv + (c >> 2));
      } else {
        qv[c] = codes;
        if ((threadIdx.x & 3) == 0) sv[c >> 2] = static_cast<uint8_t>(byte);
      }
    }
  }
}

template <int UNROLL, bool NT>
hipError_t launch_act_quant_v(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                              int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                              hipStream_t stream) {
  const int64_t chunks = M * K / 8;
  const int64_t per_block = static_cast<int64_t>(kThreads) * UNROLL;
  const int64_t blocks = (chunks + per_block - 1) / per_block;
  dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
  hipLaunchKernelGGL((act_quant_kernel<UNROLL, NT>), grid, dim3(kThreads), 0, stream, x, q, s,
                     chunks, stride_x, stride_q, stride_s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                            int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                            hipStream_t stream) {
  // Two 16-byte chunks per lane and non-temporal stores measured best for sustained streaming
  // (inputs and outputs far larger than the last-level cache).
  return launch_act_quant_v<2, true>(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
}

}  // namespace mx
