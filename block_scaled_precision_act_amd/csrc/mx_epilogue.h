// Elementwise epilogue arithmetic shared by the GEMM kernels: what is applied to the fp32 value
// (sum + bias) of one output before its single bf16 rounding.
//
// The "fp4-gemm README" page lists bias + residual and bias + GELU GEMM epilogues (so that a
// GEMM's output feeds the next low-bit GEMM without a separate elementwise pass) but gives no
// formula; here the residual is a bf16 tensor added in fp32 like the bias, and GELU is the exact
// x * Phi(x) with Phi the standard normal CDF.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mx {

// fp32 value of a bf16 bit pattern (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// x * Phi(x), without a branch.  Phi(-|x|) = erfc(z) / 2 with z = |x| / sqrt 2, and erfc is
// taken in the form of the erfcc routine of Numerical Recipes (Press et al., 2nd ed., section
// 6.2): erfc(z) = t exp(-z^2 + Q(t)), t = 1 / (1 + p z), here with p = 0.4 and a degree-4 Q
// least-squares fitted to log(exp(z^2) erfc(z) / t) over z >= 0.  Its relative error is below
// 1.2e-4 for every z >= 0, so x * Phi(x) keeps that relative accuracy for both signs and deep into
// the left tail (checked against the exact value on 34 M float32 inputs, every bf16 value among
// them); the bf16 rounding (2^-9) dominates.
// The exponent is taken in base 2 with log2(e), the 1/2 and a 2^32 pre-scale folded into Q's
// coefficients, so Phi(-|x|) * 2^32 stays a normal number until the final product: outputs as
// small as 2^-126 come out right even where Phi(-|x|) itself is below the fp32 normal range.
__device__ __forceinline__ float gelu_f32(float x) {
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(x), 0.282842726f, 1.0f));   // p / sqrt 2
  float q = -0.415893883f;
  q = fmaf(q, t, 0.610183597f);
  q = fmaf(q, t, 0.5003317f);
  q = fmaf(q, t, 1.45326746f);
  q = fmaf(q, t, 28.8521538f);           // log2(e) Q(t) - 1 + 32
  // -z^2 log2(e) = -x^2 log2(e) / 2
  const float th = t * __builtin_amdgcn_exp2f(fmaf(x * x, -0.721347511f, q));   // 2^32 Phi(-|x|)
  return x >= 0.0f ? fmaf(-x, th * 0x1p-32f, x) : (x * th) * 0x1p-32f;
}

}  // namespace mx
