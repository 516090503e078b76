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
    const uint64_t h0 = __umul64hi(kM0, x0), l0 = kM0 * x0;
    const uint64_t h1 = __umul64hi(kM1, x2), l1 = kM1 * x2;
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
