// Block-scaled GEMM with both operands MXFP4 (E2M1 + per-32 E8M0) for gfx950 on
// v_mfma_scale_f32_32x32x64_f8f6f4.  E2M1 values have at most 2 significant bits and span under
// 4 binades, so the products of one scaled MFMA fit its internal adder window and the result is
// the fp32 accumulation of exact products (measured on the device); operands with E4M3 values
// go through the bf16 path instead.
//
// C[m,n] = bf16_rne(sum_k A[m,k] B[n,k] + bias[n]) with fp32 accumulation on the matrix cores
// ("formats.py" page: decode_fp4 / decode_fp8_block / act_qdq give the decoded operands;
// "AstrAI commit log" page: the bias is added in fp32 before the single bf16 rounding).
//
// Operand registers of the scaled 32x32x64 MFMA (wave64), as measured on gfx950:
//   lane l holds row (l % 32) of A (column l % 32 of B^T) and works on half h = l / 32 of the
//   64-wide K step:
//     FP8 : 32 bytes = K [16h, 16h+16) in dwords 0..3 and K [32+16h, 32+16h+16) in dwords 4..7
//     FP4 : 16 bytes = K [32h, 32h+32) in dwords 0..3, low nibble first
//   the E8M0 byte lane l passes scales logical K-block h (K [32h, 32h+32)) of its row.
//   accumulator register r of lane l is C[8*(r/4) + 4*h + (r%4)][l % 32].
#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kUnitScale = 127u;   // E8M0 byte of 1.0, used for K-blocks past the end

struct Args {
  const uint8_t* a;
  const uint8_t* a_s;
  const uint8_t* b;
  const uint8_t* b_s;
  const uint16_t* bias;
  uint16_t* c;
  int M, N, K;
  int64_t stride_a, stride_as, stride_b, stride_bs, stride_bias, stride_c;
};

__device__ __forceinline__ uint16_t to_bf16(float v) {
  bf16x2 p = {static_cast<__bf16>(v), static_cast<__bf16>(0.0f)};
  return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, p) & 0xFFFFu);
}

// Loads lane's operand registers for the 64-wide K step starting at k0 of row `row`.
// kb_total = K / 32.  K-blocks at or past kb_total load zeros (with scale 1.0).
template <int FMT>
__device__ __forceinline__ v8i load_operand(const uint8_t* row_ptr, int k0, int h, int kb_total) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  const int kb0 = k0 / 32;            // first K-block of this step
  if (FMT == kFp8) {
    // dwords 0..3: K [k0+16h, +16) lies in block kb0 (always valid when the step starts).
    uint4 lo = *reinterpret_cast<const uint4*>(row_ptr + k0 + 16 * h);
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    if (kb0 + 1 < kb_total) {
      uint4 hi = *reinterpret_cast<const uint4*>(row_ptr + k0 + 32 + 16 * h);
      r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    }
  } else {
    if (kb0 + h < kb_total) {
      uint4 lo = *reinterpret_cast<const uint4*>(row_ptr + (k0 + 32 * h) / 2);
      r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    }
  }
  return r;
}

// One wavefront per 32x32 output tile, four wavefronts (2 x 2) per workgroup.
template <int AF, int BF, bool BIAS>
__global__ __launch_bounds__(256) void gemm_simple_kernel(Args p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int64_t bz = blockIdx.z;
  if (m0 >= p.M || n0 >= p.N) return;

  const int kb_total = p.K / 32;
  const int row_a = min(m0 + (lane & 31), p.M - 1);
  const int row_b = min(n0 + (lane & 31), p.N - 1);
  const int a_pitch = AF == kFp8 ? p.K : p.K / 2;
  const int b_pitch = BF == kFp8 ? p.K : p.K / 2;
  const uint8_t* a_row = p.a + bz * p.stride_a + static_cast<int64_t>(row_a) * a_pitch;
  const uint8_t* b_row = p.b + bz * p.stride_b + static_cast<int64_t>(row_b) * b_pitch;
  const uint8_t* as_row = p.a_s + bz * p.stride_as + static_cast<int64_t>(row_a) * kb_total;
  // FP8 B: one scale per 32x32 block -> scale row n/32; FP4 B: one scale per 32 K of row n.
  const uint8_t* bs_row = p.b_s + bz * p.stride_bs +
      static_cast<int64_t>(BF == kFp8 ? row_b / 32 : row_b) * kb_total;

  v16f acc = {};
  for (int k0 = 0; k0 < p.K; k0 += 64) {
    const int kb = k0 / 32 + h;
    v8i av = load_operand<AF>(a_row, k0, h, kb_total);
    v8i bv = load_operand<BF>(b_row, k0, h, kb_total);
    const int sa = kb < kb_total ? as_row[kb] : kUnitScale;
    const int sb = kb < kb_total ? bs_row[kb] : kUnitScale;
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, AF, BF, 0, sa, 0, sb);
  }

  const int col = n0 + (lane & 31);
  if (col >= p.N) return;
  float bias = 0.0f;
  if (BIAS) bias = __uint_as_float(static_cast<uint32_t>(p.bias[bz * p.stride_bias + col]) << 16);
  uint16_t* c = p.c + bz * p.stride_c;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + 8 * (r / 4) + 4 * h + (r % 4);
    if (row < p.M) c[static_cast<int64_t>(row) * p.N + col] = to_bf16(acc[r] + bias);
  }
}

template <int AF, int BF>
hipError_t launch_formats(const GemmProblem& g, hipStream_t stream) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c};
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch);
  if (g.bias)
    hipLaunchKernelGGL((gemm_simple_kernel<AF, BF, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_simple_kernel<AF, BF, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp4_mfma(const GemmProblem& p, hipStream_t stream) {
  return launch_formats<kFp4, kFp4>(p, stream);
}

hipError_t launch_gemm(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                       hipStream_t stream) {
  if (a_fmt == kFp4 && b_fmt == kFp4) return launch_gemm_fp4_mfma(p, stream);
  return launch_gemm_bf16(a_fmt, b_fmt, p, dev, stream);
}

}  // namespace mx
