// Pieces shared by the GEMM kernels with FP8 operands (gemm_bf16.hip, gemm_mx.hip): operand
// decoders, buffer resources, the workgroup -> tile map, and the split-K handoff plus epilogue
// that run after a main loop.
#pragma once

#include "mx_epilogue.h"
#include "mx_internal.h"
#include "mx_quant.h"

namespace mx {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <int V>
struct IntC { static constexpr int value = V; };

// Calls f(IntC<I>{}) for I in [B, E), unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt operand that waits for every vector-memory access of the wavefront (vmcnt 0) and
// for nothing else (expcnt and lgkmcnt at their maxima): vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[15:14] in the gfx9 encoding.
constexpr int kVmcntZero = 0x0F70;

struct Args {
  const uint8_t* a;
  const uint8_t* a_s;
  const uint8_t* b;
  const uint8_t* b_s;
  const uint16_t* bias;
  uint16_t* c;
  int M, N, K;
  int tiles_m, tiles_n;
  int64_t stride_a, stride_as, stride_b, stride_bs, stride_bias, stride_c;
  uint8_t* q;
  uint8_t* qs;
  int64_t stride_q, stride_qs;
  const uint16_t* res;
  int64_t stride_res;
  // SPLIT: K split into `splits` equal ranges of K steps per tile; fp32 partial tiles in `ws`
  // (tile-major, then range), one arrival counter per tile in `counters` (zero between calls).
  float* ws;
  uint32_t* counters;
  int splits;
};

// fp32 value of an E8M0 byte (2^(b-127)); byte 0 is the fp32 subnormal 2^-127.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __uint_as_float(max(b << 23, 0x00400000u));
}

__device__ __forceinline__ uint32_t pk_bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// 8 E2M1 codes (one dword, low nibble first) times s -> 8 bf16.
__device__ __forceinline__ uint4 decode_fp4_dword(uint32_t d, float s) {
  uint4 o;
  o.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0));
  o.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1));
  o.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2));
  o.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3));
  return o;
}

// 8 E4M3 codes (two dwords) times s -> 8 bf16.
__device__ __forceinline__ uint4 decode_fp8_pair(uint32_t lo, uint32_t hi, float s) {
  uint4 o;
  o.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, false));
  o.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, true));
  o.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, false));
  o.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, true));
  return o;
}

// 8 E5M2 codes (two dwords) times s -> 8 bf16.
__device__ __forceinline__ uint4 decode_bf8_pair(uint32_t lo, uint32_t hi, float s) {
  uint4 o;
  o.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, s, false));
  o.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, s, true));
  o.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, s, false));
  o.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, s, true));
  return o;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // Raw buffer (stride 0) with a byte bound: loads at or past `bytes` return zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

constexpr int kGroupM = 8;

// Tile coordinates of workgroup `bid` out of `nb`: XCD-contiguous, then grouped by kGroupM rows.
__device__ __forceinline__ void tile_of(int bid, int nb, int tiles_m, int tiles_n, int& tm, int& tn) {
  int id = bid;
  if ((nb & 7) == 0) id = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int g = id / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_g = id - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

// Tile coordinates of split tile `t` (workgroups 2 t and 2 t + 1 take its two K ranges).
// Workgroups are dealt to the 8 XCDs in turn (workgroup b to XCD b % 8), so XCD x runs range
// x % 2 of the tiles t = 4 j + x / 2.  With two ranges and a tile count divisible by 4, tile t is
// renumbered so that XCDs 2 q and 2 q + 1 hold the q-th quarter of the tiles in row-major order:
// a band of whole tile rows, whose A panels (the larger operand of a down-projection) then come
// through one XCD's L2 for each range instead of four.  Otherwise the plain tile map.
__device__ __forceinline__ void split_tile_of(int t, int nt, int splits, int tiles_m, int tiles_n,
                                              int& tm, int& tn) {
  if (splits == 2 && (nt & 3) == 0) {
    const int r = (t & 3) * (nt >> 2) + (t >> 2);
    tm = r / tiles_n;
    tn = r % tiles_n;
  } else {
    tile_of(t, nt, tiles_m, tiles_n, tm, tn);
  }
}

// Place of 16-byte chunk c of row r in the epilogue's bf16 LDS tile of CPR chunks a row: c XOR
// a few bits of r (rows 16 apart share the pattern).  The XOR is its own inverse, so the same
// function maps a stored place back to the chunk it holds.
template <int CPR>
__device__ __forceinline__ int tile_chunk(int r, int c) {
  static_assert(CPR % 4 == 0, "tile width");
  if constexpr (CPR % 16 == 0) return c ^ (r & 15);
  else if constexpr (CPR % 8 == 0) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);
}

// After the main loop: for SPLIT, the partial-tile handoff (a workgroup whose range arrived first
// returns); then the epilogue of one BM x BN tile from the accumulators of its WM x WN wavefronts:
// fp32 + bias (+ residual, or GELU), one bf16 rounding, staged through LDS rows given by
// tile_row(r) (BN * 2 bytes each, free for reuse: every wavefront is past its last operand read),
// copied out with 16-byte stores; or, QUANT, the bf16 values quantized per 32 columns straight
// from the accumulators.
// lds_bias holds the tile's BN bias values as fp32 when has_bias.  res_in_lds (residual epilogue):
// the main loop has already copied the residual tile into the LDS tile, in its layout, and every
// wavefront has waited for its own copies; the barrier below makes them visible.
template <int AF, bool QUANT, int EPI, bool SPLIT, int BM, int BN, int WM, int WN, class RowPtr>
__device__ __forceinline__ void finish_tile(const Args& p, v16f (&acc)[BM / WM / 32][BN / WN / 32],
                                            RowPtr tile_row, const float* lds_bias, bool has_bias,
                                            int split, int tile_id, int m0, int n0, int64_t bz,
                                            bool res_in_lds = false) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;
  // SPLIT: where the second range finds the first one's partial tile; the epilogue adds it
  // (unit (i * TN + j) * 4 + r4 holds the four values acc[i][j][4 r4 .. 4 r4 + 3]).
  __amdgpu_buffer_rsrc_t part_rsrc = make_rsrc(nullptr, 0);
  uint32_t part_lane = 0;
  bool part_lost = false;       // the wait gave up: the tile is written as NaN
  if constexpr (SPLIT) {
    // Two K ranges per tile, one workgroup each.  Each workgroup takes its arrival number at the
    // tile's counter as soon as its main loop is done.  The first to arrive stores its fp32
    // partial tile and then raises the tile's ready flag; the second waits for the flag, resets
    // counter and flag for the next call, loads that partial, adds it to its own accumulators
    // and runs the epilogue.  Only one partial per tile is written and read.  The wait cannot
    // hang: the workgroup it waits for is running (it has arrived) and waits for nothing.
    // Partial layout: thread t's accumulator values as 16-byte units u at (u * NT + t), so every
    // store and load is one coalesced 1 KB row per wavefront; stored and loaded with
    // device-scope cache policy (sc1), so they do not sit dirty in one XCD's L2.
    constexpr int kUnits = TM * TN * 4;
    constexpr uint32_t kTileBytes = static_cast<uint32_t>(kUnits) * NT * 16;
    constexpr int kDeviceScope = 16;     // the sc1 cache-policy bit
    constexpr uint32_t kMaxPolls = 1u << 22;
    const __amdgpu_buffer_rsrc_t wsr = make_rsrc(
        reinterpret_cast<const uint8_t*>(p.ws) + static_cast<int64_t>(tile_id) * kTileBytes,
        kTileBytes);
    uint32_t* const counter = p.counters + tile_id;
    uint32_t* const flag = p.counters + p.tiles_m * p.tiles_n + tile_id;
    const uint32_t lane_off = threadIdx.x * 16u;
    __shared__ uint32_t role;
    if (threadIdx.x == 0)
      role = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (role == 0) {
      static_for<0, TM * TN>([&](auto bc) {
        constexpr int b = decltype(bc)::value, i = b / TN, j = b % TN;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t off = static_cast<uint32_t>((b * 4 + q) * NT * 16) + lane_off;
          const v4f v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), wsr, off, 0,
                                                 kDeviceScope);
        }
      });
      // Publish.  (1) Every wavefront waits until its own partial stores are complete (vmcnt 0:
      // acknowledged by this XCD's L2): a workgroup barrier alone does not wait for stores in
      // flight, and the release below waits only for thread 0's wavefront.  (2) The barrier:
      // past it, every store of the workgroup is in the L2.  (3) Thread 0's device-scope release
      // writes this XCD's L2 back (every wavefront's partial included, by (1)), waits for the
      // write-back to finish, and only then sets the flag.
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
      __syncthreads();
      if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    // Second: wait for the flag, then acquire (this XCD's L2 drops lines it may hold stale), so
    // the loads below, ordered after it by the barrier, see the whole partial.  A wait longer
    // than ~2^22 polls (far beyond any real one) gives up and poisons the tile with NaN instead
    // of hanging.
    if (threadIdx.x == 0) {
      uint32_t polls = 0;
      while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u &&
             ++polls < kMaxPolls)
        __builtin_amdgcn_s_sleep(4);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      role = polls < kMaxPolls ? 1u : 2u;
      __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    part_rsrc = wsr;
    part_lane = lane_off;
    part_lost = role != 1u;
  }

  if constexpr (QUANT) {
    // The quantized output, straight from the accumulators (no LDS staging).  Per 32-column
    // block j of row 32 i + l32: lane (l32, h) holds the block's columns 8 r4 + 4 h + k
    // (r4, k < 4), 16 of its 32 values, and lane l32 + 32 (h flipped) holds the other 16.  Each
    // value is (sum + bias), GELU'd for EPI == kEpiGelu, rounded to bf16 once, exactly as the
    // bf16 output would hold it; the block's largest |bf16| is the max of the two lanes' maxima
    // (one exchange across the wavefront halves), and the codes are those act_quant gives for
    // those bf16 values (the same arithmetic, mx_quant.h).  A second exchange hands each lane a
    // contiguous half of the block's codes: 16 bytes (E4M3) or 8 (E2M1) per store; lane h = 0
    // stores the block's E8M0 byte.  N % 32 == 0, so a block is inside the matrix or wholly
    // outside it.
    uint8_t* q = p.q + bz * p.stride_q;
    uint8_t* qs = p.qs + bz * p.stride_qs;
    const int nb = p.N / 32;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int bcol = wn * WTN + 32 * j;                 // the block's first tile column
      const int col0 = n0 + bcol;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = m0 + wm * WTM + 32 * i + l32;
        const bool live = row < p.M && col0 < p.N;
        uint32_t lo[4], hi[4];           // bf16 pairs of columns 8 r4 + 4 h + (0, 1) and (2, 3)
        uint32_t amax = 0;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          v4f bias4 = {0.0f, 0.0f, 0.0f, 0.0f};
          if (has_bias) bias4 = *reinterpret_cast<const v4f*>(lds_bias + bcol + 8 * r4 + 4 * h);
          float v[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[k] = acc[i][j][4 * r4 + k] + bias4[k];
            if constexpr (EPI == kEpiGelu) v[k] = gelu_f32(v[k]);
          }
          lo[r4] = pk_bits(bf16x2{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])});
          hi[r4] = pk_bits(bf16x2{static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])});
          amax = max(amax, abs_max_bits(uint4{lo[r4], hi[r4], 0u, 0u}));
        }
        amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 32)));
        if constexpr (AF == kFp4) {
          const uint32_t byte = fp4_scale_byte(amax);
          const float sc = __uint_as_float(byte << 23);              // 2^E, a normal fp32
          uint32_t c[4];                                              // 4 codes = 16 bits each
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) c[r4] = encode4_fp4(lo[r4], hi[r4], sc);
          // h = 0 keeps columns 0-15 of the block (bytes 0-7), h = 1 columns 16-31 (bytes 8-15)
          const uint32_t mine_lo = c[0] | (c[1] << 16), mine_hi = c[2] | (c[3] << 16);
          const uint32_t got = static_cast<uint32_t>(
              __shfl_xor(static_cast<int>(h ? mine_lo : mine_hi), 32));
          const uint2 out = h ? uint2{(got & 0xFFFFu) | (c[2] << 16), (got >> 16) | (c[3] << 16)}
                              : uint2{c[0] | (got << 16), c[1] | (got & 0xFFFF0000u)};
          if (live) {
            *reinterpret_cast<uint2*>(q + static_cast<int64_t>(row) * (p.N / 2) + col0 / 2 + 8 * h) = out;
            if (h == 0) qs[static_cast<int64_t>(row) * nb + (col0 >> 5)] = static_cast<uint8_t>(byte);
          }
        } else {
          const uint32_t byte = act_scale_byte(amax);
          const float inv_s = __uint_as_float((254u - byte) << 23);  // 2^-E, a normal fp32
          uint32_t d[4];                                              // 4 codes each
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) d[r4] = encode4(lo[r4], hi[r4], inv_s);
          // h = 0 keeps columns 0-15 (dwords of r4 = 0, 1 and the partner's), h = 1 columns 16-31
          const uint32_t ga = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h ? d[0] : d[2]), 32));
          const uint32_t gb = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h ? d[1] : d[3]), 32));
          const uint4 out = h ? uint4{ga, d[2], gb, d[3]} : uint4{d[0], ga, d[1], gb};
          if (live) {
            *reinterpret_cast<uint4*>(q + static_cast<int64_t>(row) * p.N + col0 + 16 * h) = out;
            if (h == 0) qs[static_cast<int64_t>(row) * nb + (col0 >> 5)] = static_cast<uint8_t>(byte);
          }
        }
      }
    }
    return;
  }
  // Epilogue, staged through LDS: fp32 + bias, one bf16 rounding, written into a row-major bf16
  // tile [BM][BN], then copied out in coalesced 16-byte row segments.  The MFMA takes B as its
  // first operand, so accumulator block (i, j) holds C^T: element 4 r4 + k of a lane is row
  // 32 i + l32 and column 32 j + 8 r4 + 4 h + k of the wavefront tile, four consecutive
  // columns of one row, written to LDS as one 8-byte store.  16-byte chunk c of tile row r sits
  // at chunk tile_ch(r, c), c XOR a few bits of r: the 16 rows that 16 lanes write in one pass
  // land in 16 different 16-byte bank groups (for 28-chunk rows, of 448 bytes, rows r and r + 1
  // start 64 bytes of banks apart and the XOR of (r >> 2) & 3 does the rest), and a row's chunks
  // stay a permutation of themselves for the copy-out.
  __syncthreads();                       // every wavefront is done reading the operand stages
  constexpr int kChunksPerRow = BN / 8;
  static_assert(kChunksPerRow % 4 == 0, "tile width");
  auto tile_ch = [](int r, int c) { return tile_chunk<kChunksPerRow>(r, c); };
  if constexpr (EPI == kEpiResidual) {
    // The residual tile is first copied into the LDS tile in the same layout, with coalesced
    // 16-byte loads (zeros outside the matrix); each thread below reads the residual at its own
    // outputs' places and overwrites them with the results.  The residual may be the output
    // itself: every read of the tile precedes the barrier before the copy-out.
    const uint16_t* res = p.res + bz * p.stride_res;
    constexpr int kResIters = BM * kChunksPerRow / NT;
    static_assert((BM * kChunksPerRow) % NT == 0, "residual chunks");
    if (!res_in_lds) {
      if (m0 + BM <= p.M && n0 + BN <= p.N && (p.N & 7) == 0 &&
          (reinterpret_cast<uintptr_t>(res) & 15u) == 0) {
        // A tile inside a residual whose rows are 16-byte aligned: every thread loads all its
        // chunks (chunk threadIdx + NT it of the tile, row-major) before storing any of them, so
        // the loads are in flight together instead of one memory round trip per chunk.
        uint4 v[kResIters];
#pragma unroll
        for (int it = 0; it < kResIters; ++it) {
          const int idx = static_cast<int>(threadIdx.x) + it * NT;
          const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
          v[it] = *reinterpret_cast<const uint4*>(res + static_cast<int64_t>(m0 + trow) * p.N + n0 +
                                                  tch * 8);
        }
#pragma unroll
        for (int it = 0; it < kResIters; ++it) {
          const int idx = static_cast<int>(threadIdx.x) + it * NT;
          const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
          *reinterpret_cast<uint4*>(tile_row(trow) + tile_ch(trow, tch) * 16) = v[it];
        }
      } else {
        for (int idx = threadIdx.x; idx < BM * kChunksPerRow; idx += NT) {
          const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
          const int row = m0 + trow, col = n0 + tch * 8;
          const int ch = tile_ch(trow, tch);
          uint4 v = {0u, 0u, 0u, 0u};
          if (row < p.M && col < p.N) {
            const uint16_t* src = res + static_cast<int64_t>(row) * p.N + col;
            if (col + 8 <= p.N && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
              v = *reinterpret_cast<const uint4*>(src);
            } else {
              uint32_t e[8];
#pragma unroll
              for (int k = 0; k < 8; ++k) e[k] = col + k < p.N ? src[k] : 0u;
              v = uint4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                        e[6] | (e[7] << 16)};
            }
          }
          *reinterpret_cast<uint4*>(tile_row(trow) + ch * 16) = v;
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int tcol = wn * WTN + 32 * j + 8 * r4 + 4 * h;        // columns tcol .. tcol + 3
      v4f bias4 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (has_bias)
        bias4 = *reinterpret_cast<const v4f*>(lds_bias + tcol);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int trow = wm * WTM + 32 * i + l32;
        uint8_t* const dst = tile_row(trow) + (tile_ch(trow, tcol >> 3) * 16 + (tcol & 7) * 2);
        float v[4];
        if constexpr (SPLIT) {
          // fp32 addition is commutative, so the sum is the same bits whichever range came first
          const uint32_t off = static_cast<uint32_t>(((i * TN + j) * 4 + r4) * NT * 16) + part_lane;
          const v4f pv = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                     part_rsrc, off, 0, 16 /* sc1 */));
#pragma unroll
          for (int k = 0; k < 4; ++k)
            v[k] = part_lost ? __builtin_nanf("") : (acc[i][j][4 * r4 + k] + pv[k]) + bias4[k];
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = acc[i][j][4 * r4 + k] + bias4[k];
        }
        if constexpr (EPI == kEpiResidual) {
          const uint2 r = *reinterpret_cast<const uint2*>(dst);
          v[0] += bf16_bits_to_f32(r.x & 0xFFFFu);
          v[1] += bf16_bits_to_f32(r.x >> 16);
          v[2] += bf16_bits_to_f32(r.y & 0xFFFFu);
          v[3] += bf16_bits_to_f32(r.y >> 16);
        } else if constexpr (EPI == kEpiGelu) {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = gelu_f32(v[k]);
        }
        const bf16x2 lo = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])};
        const bf16x2 hi = {static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
        *reinterpret_cast<uint2*>(dst) = uint2{pk_bits(lo), pk_bits(hi)};
      }
    }
  }
  __syncthreads();
  {
    uint16_t* c = p.c + bz * p.stride_c;
    // A tile wholly inside an output whose rows are 16-byte aligned: thread t copies chunks
    // t + NT it of the tile (row-major, so a wavefront's stores cover whole row segments), all LDS
    // reads issued before the stores.
    constexpr int kIters = BM * kChunksPerRow / NT;
    static_assert((BM * kChunksPerRow) % NT == 0, "copy-out chunks");
    if (m0 + BM <= p.M && n0 + BN <= p.N && (p.N & 7) == 0 &&
        (reinterpret_cast<uintptr_t>(c) & 15u) == 0) {
      uint4 v[kIters];
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
        v[it] = *reinterpret_cast<const uint4*>(tile_row(trow) + tile_ch(trow, tch) * 16);
      }
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
        __builtin_nontemporal_store(__builtin_bit_cast(v4u, v[it]), reinterpret_cast<v4u*>(
            c + static_cast<int64_t>(m0 + trow) * p.N + n0 + tch * 8));
      }
    } else {
      for (int idx = threadIdx.x; idx < BM * kChunksPerRow; idx += NT) {
        const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
        const int row = m0 + trow, col = n0 + tch * 8;
        if (row >= p.M || col >= p.N) continue;
        const int ch = tile_ch(trow, tch);
        const uint4 v = *reinterpret_cast<const uint4*>(tile_row(trow) + ch * 16);
        uint16_t* dst = c + static_cast<int64_t>(row) * p.N + col;
        if (col + 8 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
            if (col + k < p.N) dst[k] = static_cast<uint16_t>((k & 1) ? w >> 16 : w);
          }
        }
      }
    }
  }
}

}  // namespace
}  // namespace mx
