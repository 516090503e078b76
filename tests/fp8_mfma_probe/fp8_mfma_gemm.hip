// TEST INFRASTRUCTURE ONLY: not part of the library.  A plain GEMM on gfx950's scaled FP8 matrix
// instruction (v_mfma_scale_f32_32x32x64_f8f6f4), written to show on the device whether that
// instruction can carry the block-scaled GEMM's accuracy bound
//   |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k|
// on the configurations' operands.  The library's FP8 GEMMs decode to exact bf16 and use the
// bf16 MFMA instead; this kernel exists only so that the reason can be re-checked.
//
// What it computes is the library's GEMM ("formats.py" page: the decoded operand is code value
// times 2^(scale byte - 127), per 32 consecutive K of a row, or per 32x32 block of an E4M3
// weight; "AstrAI commit log" page: the bias joins the fp32 sum, then one bf16 rounding):
//   c_f32[m, n] = sum_k A[m,k] B[n,k]  (the instruction's fp32 accumulation)
//   c_bf16[m, n] = bf16_rne(c_f32[m, n] + bias[n])
// A: E4M3 codes [M, K] + E8M0 [M, K/32].  B: E4M3 [N, K] + E8M0 [N/32, K/32] (b_fmt 0), or packed
// E2M1 [N, K/2] (low nibble first) + E8M0 [N, K/32] (b_fmt 4).  M % 32 == N % 32 == K % 64 == 0.
//
// One wavefront per 32x32 output block, no LDS.  Operand registers of the instruction (measured
// on gfx950): lane l holds row l % 32 of its operand, group h = l / 32.  An E4M3 lane holds K
// [16h, 16h + 16) of the 64-wide step in dwords 0..3 and K [32 + 16h, 32 + 16h + 16) in dwords
// 4..7; an E2M1 lane holds K [32h, 32h + 32) in dwords 0..3 (low nibble first).  The E8M0 byte
// lane (r, h) passes scales the 32-block h of row r.  Accumulator register j of lane l is output
// row 8 (j / 4) + 4 h + j % 4, column l % 32 of the block.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const bf16x2 p = {static_cast<__bf16>(v), static_cast<__bf16>(0.0f)};
  return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, p) & 0xFFFFu);
}

template <int BF>
__global__ __launch_bounds__(64) void fp8_mfma_gemm_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_s, const uint8_t* __restrict__ b,
    const uint8_t* __restrict__ b_s, const uint16_t* __restrict__ bias, uint16_t* __restrict__ c,
    float* __restrict__ c_f32, int M, int N, int K) {
  const int lane = threadIdx.x;
  const int r = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int kb = K / 32;
  const uint8_t* arow = a + static_cast<int64_t>(m0 + r) * K;
  v16f acc = {};
  for (int k0 = 0; k0 < K; k0 += 64) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(arow + k0 + 16 * h);
    const uint4 a1 = *reinterpret_cast<const uint4*>(arow + k0 + 32 + 16 * h);
    const v8i av = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                    static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                    static_cast<int>(a1.z), static_cast<int>(a1.w)};
    const int sa = a_s[static_cast<int64_t>(m0 + r) * kb + k0 / 32 + h];
    v8i bv;
    int sb;
    if constexpr (BF == 0) {
      const uint8_t* brow = b + static_cast<int64_t>(n0 + r) * K;
      const uint4 b0 = *reinterpret_cast<const uint4*>(brow + k0 + 16 * h);
      const uint4 b1 = *reinterpret_cast<const uint4*>(brow + k0 + 32 + 16 * h);
      bv = v8i{static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
               static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
               static_cast<int>(b1.z), static_cast<int>(b1.w)};
      sb = b_s[static_cast<int64_t>((n0 + r) / 32) * kb + k0 / 32 + h];
    } else {
      const uint8_t* brow = b + static_cast<int64_t>(n0 + r) * (K / 2);
      const uint4 b0 = *reinterpret_cast<const uint4*>(brow + (k0 + 32 * h) / 2);
      bv = v8i{static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
               static_cast<int>(b0.w), 0, 0, 0, 0};
      sb = b_s[static_cast<int64_t>(n0 + r) * kb + k0 / 32 + h];
    }
    // A format 0 (E4M3), B format BF (0: E4M3, 4: E2M1); byte 0 of each scale register
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, BF, 0, sa, 0, sb);
  }
  const int col = n0 + r;
  const float bv = bias ? __uint_as_float(static_cast<uint32_t>(bias[col]) << 16) : 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = m0 + 8 * (j / 4) + 4 * h + (j % 4);
    const int64_t o = static_cast<int64_t>(row) * N + col;
    c_f32[o] = acc[j];
    c[o] = bf16_rne(acc[j] + bv);
  }
}

}  // namespace

extern "C" {

// Returns 0 on success, -2 for a shape this kernel does not take, -6 when the launch failed.
int fp8_mfma_probe_gemm(int b_fmt, const void* a, const void* a_s, const void* b, const void* b_s,
                        const void* bias, void* c_bf16, void* c_f32, int64_t M, int64_t N,
                        int64_t K, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0 || M % 32 || N % 32 || K % 64 || M > 65535 * 32 ||
      N > (int64_t{1} << 26) || M * K >= (int64_t{1} << 31) || N * K >= (int64_t{1} << 31) ||
      M * N >= (int64_t{1} << 31) || (b_fmt != 0 && b_fmt != 4))
    return -2;
  const dim3 grid(static_cast<unsigned>(N / 32), static_cast<unsigned>(M / 32));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  auto* pa = static_cast<const uint8_t*>(a);
  auto* pas = static_cast<const uint8_t*>(a_s);
  auto* pb = static_cast<const uint8_t*>(b);
  auto* pbs = static_cast<const uint8_t*>(b_s);
  auto* pbias = static_cast<const uint16_t*>(bias);
  auto* pc = static_cast<uint16_t*>(c_bf16);
  auto* pf = static_cast<float*>(c_f32);
  if (b_fmt == 0)
    hipLaunchKernelGGL(fp8_mfma_gemm_kernel<0>, grid, dim3(64), 0, s, pa, pas, pb, pbs, pbias, pc,
                       pf, m, n, k);
  else
    hipLaunchKernelGGL(fp8_mfma_gemm_kernel<4>, grid, dim3(64), 0, s, pa, pas, pb, pbs, pbias, pc,
                       pf, m, n, k);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
