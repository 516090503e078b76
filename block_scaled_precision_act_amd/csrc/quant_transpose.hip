// Quantize-transpose for gfx950: bf16 x [R, C] -> codes [C, R] + E8M0 bytes [C, R/32], the 32-blocks
// running along R, so that the transpose of x is ready as a GEMM operand whose contraction is R.
// The hip_quant page offers fused quantize-plus-transpose for rank-2 tensors (no full-precision
// transpose is materialized), and the AstrAI page routes the input and weight gradients of a
// linear layer through the forward GEMM on transposed operands: dX = dY W reads W^T quantized
// along N, dW = dY^T X reads dY^T and X^T quantized along the tokens.
//   E4M3 (fmt kFp8): the act_quant rule (the "formats.py" page's act_scale / act_quant);
//   E5M2 (fmt kBf8): the gradient rule (E5M2's 57344 in that rule, amax floor 2^-126, E >= -127),
//       rounded to nearest even or stochastically; the uniform of output element i (its index
//       c * R + r in the [C, R] output) is word i & 7 of Philox4x64-10 block i >> 3.
//
// A workgroup owns a tile of 128 rows x 64 columns of x.  It is loaded with coalesced 16-byte row
// chunks into LDS; lane (column c, block b) then reads its 32 values down column c (rows
// 32b .. 32b + 31 of the tile) and writes them as 32 consecutive codes of output row c: four
// consecutive lanes write the four blocks of one output row (128 contiguous bytes).  In LDS,
// 16-byte chunk j of tile row r sits at chunk j ^ 2 ((r >> 5) & 3), so the four row blocks a
// wavefront reads at once fall in distinct banks.
#include "mx_internal.h"
#include "mx_philox.h"
#include "mx_quant.h"

namespace mx {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kTR = 128;            // tile rows (4 blocks of 32 along R)
constexpr int kTC = 64;             // tile columns
constexpr int kQThreads = 256;      // one lane per (column, block) of the tile

template <int FMT, bool STOCH>
__global__ __launch_bounds__(kQThreads) void quant_transpose_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ s, int R,
    int C, uint64_t seed) {
  __shared__ uint4 tile[kTR * kTC / 8];
  const int r0 = blockIdx.y * kTR, c0 = blockIdx.x * kTC;
  // All of a thread's loads are issued before any of them is stored to LDS (one memory round
  // trip, not one per load); a tile wholly inside the matrix loads without bounds checks.
  constexpr int kLoads = kTR * kTC / 8 / kQThreads;
  const bool whole = r0 + kTR <= R && c0 + kTC <= C;
  uint4 vin[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int idx = static_cast<int>(threadIdx.x) + i * kQThreads;
    const int r = idx >> 3, j = idx & 7;
    const int gr = r0 + r, gc = c0 + j * 8;
    vin[i] = make_uint4(0, 0, 0, 0);
    if (whole || (gr < R && gc < C))
      vin[i] = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(gr) * C + gc);
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int idx = static_cast<int>(threadIdx.x) + i * kQThreads;
    const int r = idx >> 3, j = idx & 7;
    tile[r * 8 + (j ^ (2 * ((r >> 5) & 3)))] = vin[i];
  }
  __syncthreads();

  const int c = static_cast<int>(threadIdx.x) >> 2, b = static_cast<int>(threadIdx.x) & 3;
  const int gc = c0 + c, gr0 = r0 + 32 * b;
  if (gc >= C || gr0 >= R) return;          // R % 32 == 0: a block is all in or all out
  const uint16_t* t16 = reinterpret_cast<const uint16_t*>(tile);
  const int jj = (c >> 3) ^ (2 * b);
  uint32_t v[16];                           // rows 32b + 2i, 32b + 2i + 1 of column c
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 32 * b + 2 * i;
    const uint32_t lo = t16[(r * 8 + jj) * 8 + (c & 7)];
    const uint32_t hi = t16[((r + 1) * 8 + jj) * 8 + (c & 7)];
    v[i] = lo | (hi << 16);
    amax = max(amax, max(lo & 0x7FFFu, hi & 0x7FFFu));
  }

  uint32_t out[8];                          // 32 codes, element order kept
  uint32_t byte;
  if constexpr (FMT == kFp8) {
    byte = act_scale_byte(amax);
    const float inv_s = inv_scale_of_byte(byte);
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = encode4(v[2 * k], v[2 * k + 1], inv_s);
  } else {
    byte = e5m2_scale_byte(amax);
    const float inv_s = inv_scale_of_byte(byte);
    if constexpr (STOCH) {
      const uint64_t first = (static_cast<uint64_t>(gc) * static_cast<uint64_t>(R) + gr0) >> 3;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Philox4x64Out rn = philox4x64_10(first + t, seed);
        out[2 * t] = encode4_e5m2_sr(v[4 * t], v[4 * t + 1], inv_s, philox_word(rn, 0),
                                     philox_word(rn, 1), philox_word(rn, 2), philox_word(rn, 3));
        out[2 * t + 1] = encode4_e5m2_sr(v[4 * t + 2], v[4 * t + 3], inv_s, philox_word(rn, 4),
                                         philox_word(rn, 5), philox_word(rn, 6), philox_word(rn, 7));
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) out[k] = encode4_e5m2(v[2 * k], v[2 * k + 1], inv_s);
    }
  }
  uint8_t* dst = q + static_cast<int64_t>(gc) * R + gr0;
  __builtin_nontemporal_store(v4u{out[0], out[1], out[2], out[3]}, reinterpret_cast<v4u*>(dst));
  __builtin_nontemporal_store(v4u{out[4], out[5], out[6], out[7]}, reinterpret_cast<v4u*>(dst) + 1);
  s[static_cast<int64_t>(gc) * (R / 32) + gr0 / 32] = static_cast<uint8_t>(byte);
}

template <int FMT, bool STOCH>
hipError_t launch_qt(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t R, int64_t C,
                     hipStream_t stream, uint64_t seed) {
  dim3 grid(static_cast<unsigned>((C + kTC - 1) / kTC), static_cast<unsigned>((R + kTR - 1) / kTR));
  hipLaunchKernelGGL((quant_transpose_kernel<FMT, STOCH>), grid, dim3(kQThreads), 0, stream, x, q,
                     s, static_cast<int>(R), static_cast<int>(C), seed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_transpose(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t R, int64_t C,
                                  hipStream_t stream, int fmt, bool stochastic, uint64_t seed) {
  if (fmt == kFp8) return launch_qt<kFp8, false>(x, q, s, R, C, stream, 0);
  if (stochastic) return launch_qt<kBf8, true>(x, q, s, R, C, stream, seed);
  return launch_qt<kBf8, false>(x, q, s, R, C, stream, 0);
}

}  // namespace mx
