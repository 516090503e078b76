// Internal interface between the C-ABI layer (mx_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mx {

// Operand encodings, numbered as the scaled f8f6f4 MFMA's format fields number them.
enum OperandFmt : int { kFp8 = 0, kFp4 = 4 };

// What the epilogue does to (sum + bias) before the single bf16 rounding.
enum Epilogue : int {
  kEpiPlain = 0,      // nothing
  kEpiResidual = 1,   // + residual[m, n] (bf16 [M, N])
  kEpiGelu = 2,       // x * Phi(x)
};

// One validated GEMM problem.  Per-matrix element counts are < 2^31; batch strides are in
// elements of each buffer (bytes for codes / packed / scales, bf16 elements for bias and c).
struct GemmProblem {
  const uint8_t* a;
  const uint8_t* a_s;
  const uint8_t* b;
  const uint8_t* b_s;
  const uint16_t* bias;   // nullptr: no bias
  uint16_t* c;            // bf16 output, or nullptr when the output is quantized (q, qs)
  int M, N, K, batch;
  int64_t stride_a, stride_as, stride_b, stride_bs, stride_bias, stride_c;
  uint8_t* q = nullptr;   // E4M3 codes of the bf16 output [M, N] (N % 32 == 0)
  uint8_t* qs = nullptr;  // their E8M0 bytes [M, N/32]
  int64_t stride_q = 0, stride_qs = 0;
  int epi = kEpiPlain;    // kEpiResidual / kEpiGelu: bf16 output only (q == nullptr)
  const uint16_t* residual = nullptr;   // kEpiResidual: bf16 [M, N], may be c itself
  int64_t stride_res = 0;
};

struct DeviceInfo {
  int device;
  int cu_count;
  bool gfx950;
};

// Cached per-device properties of the calling thread's current device (false: no device).
bool current_device(DeviceInfo* info);

// fmt: kFp8 (E4M3 codes [M, K]) or kFp4 (packed E2M1 [M, K/2]); scales E8M0 [M, K/32].
hipError_t launch_act_quant(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                            int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                            hipStream_t stream, int fmt = kFp8);

// FP8-operand kinds: exact bf16 decode + bf16 MFMA (gemm_bf16.hip).
hipError_t launch_gemm_bf16(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                            hipStream_t stream);
// Both operands MXFP4 on the scaled f8f6f4 MFMA (gemm_fp4.hip).
hipError_t launch_gemm_fp4_mfma(const GemmProblem& p, hipStream_t stream);

// Picks the kernel for a problem.
hipError_t launch_gemm(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                       hipStream_t stream);

}  // namespace mx
