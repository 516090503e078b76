// Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), for the stochastic rounding of gradients: a pure
// function of (counter, key), so every element's random word depends only on the seed and its
// index.  A round maps (x0, x1, x2, x3) with (h0, l0) = M0 * x0 and (h1, l1) = M1 * x2 (128-bit
// products) to (h1 ^ x1 ^ k0, l1, h0 ^ x3 ^ k1, l0); the key advances by the Weyl increments
// (W0, W1) between rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mx {

struct Philox4x64Out {
  uint64_t w[4];
};

// The full 128-bit product a * b as (hi, lo), from four 32 x 32 -> 64-bit multiply-adds: every
// partial sum fits in 64 bits, (2^32 - 1)^2 + 2 (2^32 - 1) = 2^64 - 1, so no carry is lost.
__device__ __forceinline__ void mul64_full(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint64_t a0 = static_cast<uint32_t>(a), a1 = a >> 32;
  const uint64_t b0 = static_cast<uint32_t>(b), b1 = b >> 32;
  const uint64_t p00 = a0 * b0;
  const uint64_t p01 = a0 * b1 + (p00 >> 32);
  const uint64_t p10 = a1 * b0 + static_cast<uint32_t>(p01);
  const uint64_t p11 = a1 * b1 + (p01 >> 32);
  lo = (p10 << 32) | static_cast<uint32_t>(p00);
  hi = p11 + (p10 >> 32);
}

// Block `ctr` (counter (ctr, 0, 0, 0)) under key (seed, 0).
__device__ __forceinline__ Philox4x64Out philox4x64_10(uint64_t ctr, uint64_t seed) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = ctr, x1 = 0, x2 = 0, x3 = 0, k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    uint64_t h0, l0, h1, l1;
    mul64_full(kM0, x0, h0, l0);
    mul64_full(kM1, x2, h1, l1);
    x0 = h1 ^ x1 ^ k0;
    x1 = l1;
    x2 = h0 ^ x3 ^ k1;
    x3 = l0;
  }
  return Philox4x64Out{{x0, x1, x2, x3}};
}

// 32-bit word j (0..7) of a block: 64-bit word j / 2, low half first.
__device__ __forceinline__ uint32_t philox_word(const Philox4x64Out& o, int j) {
  return static_cast<uint32_t>(o.w[j >> 1] >> (32 * (j & 1)));
}

}  // namespace mx
