// act_quant for gfx950: bf16 [M, K] -> E4M3 codes [M, K] + E8M0 scale bytes [M, K/32], the
// MXFP4 producer bf16 [M, K] -> packed E2M1 [M, K/2] + E8M0 [M, K/32], and the gradient quantizer
// bf16 [M, K] -> E5M2 codes [M, K] + E8M0 [M, K/32].
//
// Semantics: the "formats.py" page's act_scale / act_quant, per 32 consecutive elements of a row
// (the arithmetic is in mx_quant.h, shared with the quantizing GEMM epilogue); the MXFP4 producer
// applies the same rule with E2M1's largest magnitude 6 in place of 448, the gradient quantizer
// with E5M2's 57344 (hip_quant page: E5M2 for backward gradients, round-to-nearest-even or, opt-in,
// stochastic rounding from a per-element hash of (seed, index)).
//
// Bandwidth design: a row's 32-blocks are contiguous and K % 32 == 0, so a contiguous [M, K]
// matrix is one flat run of 32-blocks and scale byte i belongs to elements [32i, 32i+32).
// Each lane owns 16-byte chunks (8 bf16); the four lanes of a DPP quad own one block, so the
// block max needs two quad permutes and no LDS.  Loads are 16 B, stores of codes are 8 B per lane
// (512 contiguous bytes per wavefront), the scale byte is written by the quad's first lane.  Every
// input is read once and every output written once, so loads and stores are all non-temporal
// (streamed past the caches): on a [16384, 7168] input the non-temporal loads measured 55 us
// against 59 us for cached ones.
#include "mx_internal.h"
#include "mx_philox.h"
#include "mx_quant.h"

namespace mx {
namespace {

constexpr int kThreads = 256;

typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ void store_stream(uint2* p, uint2 v) {
  __builtin_nontemporal_store(v2u32{v.x, v.y}, reinterpret_cast<v2u32*>(p));
}

// grid.x covers ceil(chunks / (kThreads * UNROLL)) slots, grid.y is the batch index.
// UNROLL: 16-byte chunks in flight per lane.
// STOCH (E5M2 only): chunk c of batch b holds output elements 8 (b * chunks + c) + j, j < 8, whose
// uniforms are the eight 32-bit words of Philox block b * chunks + c under the seed.
template <int UNROLL, int FMT, bool STOCH = false>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ s,
    int64_t chunks, int64_t stride_x, int64_t stride_q, int64_t stride_s, uint64_t seed) {
  const int64_t bz = blockIdx.y;
  const uint4* xv = reinterpret_cast<const uint4*>(x + bz * stride_x);
  uint2* qv = reinterpret_cast<uint2*>(q + bz * stride_q);
  uint8_t* sv = s + bz * stride_s;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * UNROLL) + threadIdx.x;

  uint4 w[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t c = base + u * kThreads;
    w[u] = c < chunks ? load_stream(xv + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t c = base + u * kThreads;
    // A quad's four chunks are all in range or all out of range (chunks % 4 == 0 and quads
    // start at multiples of 4), so the quad permute inside quant_chunk only mixes live lanes.
    if constexpr (FMT == kBf8) {
      const uint32_t byte = e5m2_scale_byte(quad_max(abs_max_bits(w[u])));
      const float inv_s = inv_scale_of_byte(byte);
      uint2 codes;
      if constexpr (STOCH) {
        const Philox4x64Out r = philox4x64_10(static_cast<uint64_t>(bz * chunks + c), seed);
        codes.x = encode4_e5m2_sr(w[u].x, w[u].y, inv_s, philox_word(r, 0), philox_word(r, 1),
                                  philox_word(r, 2), philox_word(r, 3));
        codes.y = encode4_e5m2_sr(w[u].z, w[u].w, inv_s, philox_word(r, 4), philox_word(r, 5),
                                  philox_word(r, 6), philox_word(r, 7));
      } else {
        codes.x = encode4_e5m2(w[u].x, w[u].y, inv_s);
        codes.y = encode4_e5m2(w[u].z, w[u].w, inv_s);
      }
      if (c < chunks) {
        store_stream(qv + c, codes);
        if ((threadIdx.x & 3) == 0) __builtin_nontemporal_store(static_cast<uint8_t>(byte), sv + (c >> 2));
      }
      continue;
    }
    if constexpr (FMT == kFp4) {
      const QuantChunkFp4 qc = quant_chunk_fp4(w[u]);
      if (c < chunks) {
        uint32_t* q4 = reinterpret_cast<uint32_t*>(q + bz * stride_q);
        __builtin_nontemporal_store(qc.codes, q4 + c);
        if ((threadIdx.x & 3) == 0) __builtin_nontemporal_store(static_cast<uint8_t>(qc.byte), sv + (c >> 2));
      }
      continue;
    }
    const QuantChunk qc = quant_chunk(w[u]);
    if (c < chunks) {
      store_stream(qv + c, qc.codes);
      if ((threadIdx.x & 3) == 0) __builtin_nontemporal_store(static_cast<uint8_t>(qc.byte), sv + (c >> 2));
    }
  }
}

template <int UNROLL, int FMT, bool STOCH = false>
hipError_t launch_act_quant_v(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                              int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                              hipStream_t stream, uint64_t seed = 0) {
  const int64_t chunks = M * K / 8;
  const int64_t per_block = static_cast<int64_t>(kThreads) * UNROLL;
  const int64_t blocks = (chunks + per_block - 1) / per_block;
  dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
  hipLaunchKernelGGL((act_quant_kernel<UNROLL, FMT, STOCH>), grid, dim3(kThreads), 0, stream,
                     x, q, s, chunks, stride_x, stride_q, stride_s, seed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                            int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                            hipStream_t stream, int fmt, bool stochastic, uint64_t seed) {
  // Two 16-byte chunks per lane measured best for sustained streaming (inputs and outputs far
  // larger than the last-level cache).
  if (fmt == kBf8 && stochastic)
    return launch_act_quant_v<2, kBf8, true>(x, q, s, M, K, batch, stride_x, stride_q,
                                                   stride_s, stream, seed);
  if (fmt == kBf8)
    return launch_act_quant_v<2, kBf8>(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
  if (fmt == kFp4)
    return launch_act_quant_v<2, kFp4>(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
  return launch_act_quant_v<2, kFp8>(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
}

}  // namespace mx
