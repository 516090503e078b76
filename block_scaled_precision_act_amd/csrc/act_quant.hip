// act_quant for gfx950: bf16 [M, K] -> E4M3 codes [M, K] + E8M0 scale bytes [M, K/32], and the
// MXFP4 producer bf16 [M, K] -> packed E2M1 [M, K/2] + E8M0 [M, K/32].
//
// Semantics: the "formats.py" page's act_scale / act_quant, per 32 consecutive elements of a row
// (the arithmetic is in mx_quant.h, shared with the quantizing GEMM epilogue); the MXFP4 producer
// applies the same rule with E2M1's largest magnitude 6 in place of 448.
//
// Bandwidth design: a row's 32-blocks are contiguous and K % 32 == 0, so a contiguous [M, K]
// matrix is one flat run of 32-blocks and scale byte i belongs to elements [32i, 32i+32).
// Each lane owns 16-byte chunks (8 bf16); the four lanes of a DPP quad own one block, so the
// block max needs two quad permutes and no LDS.  Loads are 16 B, stores of codes are 8 B per lane
// (512 contiguous bytes per wavefront), the scale byte is written by the quad's first lane; code
// and scale stores are non-temporal (streamed past the caches).
#include "mx_internal.h"
#include "mx_quant.h"

namespace mx {
namespace {

constexpr int kThreads = 256;

// grid.x covers ceil(chunks / (kThreads * UNROLL)) slots, grid.y is the batch index.
// UNROLL: 16-byte chunks in flight per lane; NT: non-temporal code and scale stores.
template <int UNROLL, bool NT, int FMT>
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
    // start at multiples of 4), so the quad permute inside quant_chunk only mixes live lanes.
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
      if (NT) {
        __builtin_nontemporal_store(qc.codes.x, reinterpret_cast<uint32_t*>(qv + c));
        __builtin_nontemporal_store(qc.codes.y, reinterpret_cast<uint32_t*>(qv + c) + 1);
        if ((threadIdx.x & 3) == 0) __builtin_nontemporal_store(static_cast<uint8_t>(qc.byte), sv + (c >> 2));
      } else {
        qv[c] = qc.codes;
        if ((threadIdx.x & 3) == 0) sv[c >> 2] = static_cast<uint8_t>(qc.byte);
      }
    }
  }
}

template <int UNROLL, bool NT, int FMT>
hipError_t launch_act_quant_v(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                              int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                              hipStream_t stream) {
  const int64_t chunks = M * K / 8;
  const int64_t per_block = static_cast<int64_t>(kThreads) * UNROLL;
  const int64_t blocks = (chunks + per_block - 1) / per_block;
  dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
  hipLaunchKernelGGL((act_quant_kernel<UNROLL, NT, FMT>), grid, dim3(kThreads), 0, stream, x, q, s,
                     chunks, stride_x, stride_q, stride_s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                            int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                            hipStream_t stream, int fmt) {
  // Two 16-byte chunks per lane and non-temporal stores measured best for sustained streaming
  // (inputs and outputs far larger than the last-level cache).
  if (fmt == kFp4)
    return launch_act_quant_v<2, true, kFp4>(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
  return launch_act_quant_v<2, true, kFp8>(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
}

}  // namespace mx
