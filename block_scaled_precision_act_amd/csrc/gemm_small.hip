// Block-scaled GEMM with FP8 / FP4 operands for gfx950 on problems with few output tiles and a
// short K (K a multiple of 256, at most 1024): 64x64 output tiles, every K byte of the tile's
// operands copied into LDS at the start, decoded to exact bf16 in registers.
//
// What is computed is the same as in gemm_bf16.hip ("formats.py" page: decode_fp4 /
// decode_fp8_block / act_qdq give the decoded operands; "AstrAI commit log" page: the bias joins
// the fp32 sum, which is rounded to bf16 once):
//   C[m,n] = bf16_rne( sum_k A[m,k] B[n,k] + bias[n] ),
// contracted on the bf16 MFMA (v_mfma_f32_32x32x16_bf16), which forms exact products of the
// exactly decoded values and accumulates them in fp32.
//
// Why a kernel of its own: with 64x64 tiles a wavefront does only 4 MFMAs per 64-wide K step, so
// a pipeline that keeps one or two K steps of loads in flight waits for memory at every step.
// Here the whole K of the tile (at most 64 KB of A codes and 64 KB of B codes) is copied global ->
// LDS by buffer loads with the LDS as destination, all issued at the start: one memory round
// trip, then the copies stream in while the tile computes.
//   * K is cut into chunks of 256 (4 steps); chunk c goes to its own LDS array, so the
//     compiler's wait counting tells a read of chunk c from the copies of later chunks, and each
//     chunk needs one wait (vmcnt: the copies of later chunks may still be in flight) and one
//     barrier.  A row of a chunk is 256 bytes of E4M3 or 128 of E2M1, so a 1 KB copy covers 4
//     or 8 whole rows: whole 128-byte lines.  Chunks past K load zeros (every problem issues four
//     chunks of copies, so the wait counts are constants).
//   * 16-byte unit u of row r is stored at u ^ (r & 15) (256-byte rows) or u ^ ((r >> 1) & 7)
//     (128-byte rows): the 16 rows one read pass serves hit 16 different bank groups.
//   * The 4 wavefronts form a 2 x 2 grid of 32 x 32 blocks; lane group h of sub-step q of a step
//     contracts K [32h + 8q, 32h + 8q + 8) of it, for A and for B (a permutation of K, so the sum
//     is unchanged), so a lane decodes one 32-block of its row per step with one scale byte.
//   * Scale bytes: each lane loads its row's K / 32 bytes (its 32-row block's, for 32x32 block
//     scales) once, at the start, into registers.
//   * Epilogue: the one of the other GEMM kernels (gemm_common.h), staging the bf16 tile in the
//     first chunk's array.
#include "gemm_common.h"

namespace mx {
namespace {

constexpr int kSmTile = 64;
constexpr int kSmWaves = 4;
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmChunks = 4;
constexpr int kSmChunkK = 256;
constexpr uint32_t kSmOob = 0x80000000u;   // past any buffer bound

// Bytes of one operand row per chunk.
template <int FMT>
constexpr int sm_row_bytes() { return byte_codes(FMT) ? 256 : 128; }

template <int FMT>
__device__ __forceinline__ int sm_swz(int r) { return byte_codes(FMT) ? (r & 15) : ((r >> 1) & 7); }

typedef __attribute__((address_space(3))) void* sm_lds_ptr_t;

// Global -> LDS copies of one operand's 64 tile rows, one chunk at a time.  Wavefront w's copy j
// fills the KB (w * kPer + j) of the operand's region of a chunk array; lane i brings the 16 bytes
// that belong at byte 16 i of it (row and stored unit from the position, logical unit through the
// swizzle).  Rows past the matrix, and chunks past K, read zeros through the buffer bound.
template <int FMT>
struct SmCopier {
  static constexpr int kRB = sm_row_bytes<FMT>();
  static constexpr int kPer = kSmTile * kRB / 1024 / kSmWaves;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[kPer];
  uint32_t lds_off[kPer];

  __device__ __forceinline__ void init(const uint8_t* base, int row0, int rows_valid, int K,
                                       int wave, int lane, uint32_t region) {
    const uint32_t pitch = byte_codes(FMT) ? K : K / 2;
    rsrc = make_rsrc(base, static_cast<uint32_t>(rows_valid) * pitch);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int pos = (wave * kPer + j) * 1024 + 16 * lane;
      const int r = pos / kRB;
      const int u = ((pos % kRB) >> 4) ^ sm_swz<FMT>(r);
      voff[j] = row0 + r < rows_valid ? static_cast<uint32_t>(row0 + r) * pitch + 16u * u : kSmOob;
      lds_off[j] = region + static_cast<uint32_t>(wave * kPer + j) * 1024u;
    }
  }

  template <int J>
  __device__ __forceinline__ void issue(uint8_t* chunk, int c, uint32_t oob) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (sm_lds_ptr_t)(chunk + lds_off[J]), 16,
                                             static_cast<int>(voff[J] | oob), c * kRB, 0, 0);
  }
};

// One wavefront's view of one operand: the 32 rows r0 + l32 of its block.  Per step t (of the
// whole K) the lane reads the raw codes of 32-block h of its row: E4M3/E5M2 two 16-byte units,
// E2M1 one; and takes its scale byte 2t + h from the bytes loaded at the start.
template <int FMT, bool BLOCK_SCALES>
struct SmFrag {
  static constexpr int kRB = sm_row_bytes<FMT>();
  static constexpr int kUnits = byte_codes(FMT) ? 2 : 1;
  uint32_t rd[4][kUnits];    // region-relative LDS offset of unit q for step s of a chunk
  uint4 sbytes[2];           // the row's scale bytes 0..31
  uint32_t hsh;              // 8 h

  __device__ __forceinline__ void init(const uint8_t* sbase, int row0, int rows_valid, int K,
                                       int r_tile, int l32, int h, uint32_t region) {
    const int r = r_tile + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < kUnits; ++q) {
        const int u = byte_codes(FMT) ? 4 * s + 2 * h + q : 2 * s + h;
        rd[s][q] = region + static_cast<uint32_t>(r * kRB + ((u ^ sm_swz<FMT>(r)) << 4));
      }
    const int kb = K / 32;
    const int srows = BLOCK_SCALES ? (rows_valid + 31) / 32 : rows_valid;
    const int row = row0 + r;
    const int sr = BLOCK_SCALES ? row / 32 : row;
    const __amdgpu_buffer_rsrc_t srsrc =
        make_rsrc(sbase, static_cast<uint32_t>(srows) * static_cast<uint32_t>(kb));
    const uint32_t soff = sr < srows ? static_cast<uint32_t>(sr) * kb : kSmOob;
    // bytes past the row's kb belong to the next row or lie past the buffer: never used
    sbytes[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(srsrc, soff, 0, 0));
    sbytes[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              srsrc, kb > 16 ? soff : kSmOob, 16, 0));
    hsh = 8u * h;
  }

  // Scale value of step T (of the whole K): byte 2T + h.
  template <int T>
  __device__ __forceinline__ float scale() const {
    const uint4 v = sbytes[T >> 3];
    constexpr int d = (T >> 1) & 3;
    const uint32_t w = d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
    return e8m0_value((w >> (16u * (T & 1) + hsh)) & 0xFFu);
  }

  template <int S>
  __device__ __forceinline__ void read(const uint8_t* chunk, uint4 (&raw)[kUnits]) const {
#pragma unroll
    for (int q = 0; q < kUnits; ++q) raw[q] = *reinterpret_cast<const uint4*>(chunk + rd[S][q]);
  }

  // bf16 operand for sub-step Q from the raw units of a step.
  template <int Q>
  static __device__ __forceinline__ bf16x8 decode(const uint4 (&raw)[kUnits], float s) {
    uint4 o;
    if constexpr (FMT == kFp4) {
      const uint4 q = raw[0];
      o = decode_fp4_dword(Q == 0 ? q.x : Q == 1 ? q.y : Q == 2 ? q.z : q.w, s);
    } else {
      const uint4 q = raw[Q >> 1];
      const uint32_t lo = (Q & 1) ? q.z : q.x, hi = (Q & 1) ? q.w : q.y;
      o = FMT == kBf8 ? decode_bf8_pair(lo, hi, s) : decode_fp8_pair(lo, hi, s);
    }
    return __builtin_bit_cast(bf16x8, o);
  }
};

// s_waitcnt operand: vmcnt(n), lgkmcnt and expcnt at their maxima (gfx9 encoding).
constexpr int sm_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int AF, int BF, bool BIAS, bool QUANT, int EPI>
__global__ __launch_bounds__(kSmThreads) void gemm_small_kernel(Args p) {
  constexpr int kRA = sm_row_bytes<AF>(), kRBb = sm_row_bytes<BF>();
  constexpr int kBRegion = kSmTile * kRA;
  constexpr int kChunkBytes = kBRegion + kSmTile * kRBb;
  __shared__ __attribute__((aligned(16))) uint8_t ch0[kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ch1[kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ch2[kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ch3[kChunkBytes];
  __shared__ float lds_bias[kSmTile];
  uint8_t* const ch[kSmChunks] = {ch0, ch1, ch2, ch3};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t bz = blockIdx.y;
  const int m0 = tm * kSmTile, n0 = tn * kSmTile;
  const int nch = p.K / kSmChunkK;              // 1..4

  SmFrag<AF, false> fa;
  SmFrag<BF, BF == kFp8> fb;
  fa.init(p.a_s + bz * p.stride_as, m0, p.M, p.K, wm * 32, l32, h, 0);
  fb.init(p.b_s + bz * p.stride_bs, n0, p.N, p.K, wn * 32, l32, h, kBRegion);
  const bool has_bias = BIAS && (EPI == kEpiPlain || p.bias != nullptr);
  // The tile's bias, column (thread & 63), as raw bits (a buffer of no bytes without a bias: no
  // branch, so nothing waits for the load before the copies leave); threads < 64 store it.
  const __amdgpu_buffer_rsrc_t brsrc = make_rsrc(
      has_bias ? p.bias + bz * p.stride_bias : nullptr, has_bias ? 2u * p.N : 0u);
  const uint32_t bias_bits = __builtin_amdgcn_raw_buffer_load_b16(
      brsrc, 2u * min(n0 + static_cast<int>(threadIdx.x & 63), p.N - 1), 0, 0);
  // these loads stay ahead of the copies, so that the waits below count the copies alone
  __builtin_amdgcn_sched_barrier(0);

  // Every copy of the tile, chunk by chunk, behind the scale bytes.
  SmCopier<AF> ca;
  SmCopier<BF> cb;
  ca.init(p.a + bz * p.stride_a, m0, p.M, p.K, wave, lane, 0);
  cb.init(p.b + bz * p.stride_b, n0, p.N, p.K, wave, lane, kBRegion);
  constexpr int kCp = SmCopier<AF>::kPer + SmCopier<BF>::kPer;    // copies per wavefront and chunk
  static_for<0, kSmChunks>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    const uint32_t oob = c < nch ? 0u : kSmOob;
    static_for<0, SmCopier<AF>::kPer>([&](auto jc) { ca.template issue<decltype(jc)::value>(ch[c], c, oob); });
    static_for<0, SmCopier<BF>::kPer>([&](auto jc) { cb.template issue<decltype(jc)::value>(ch[c], c, oob); });
  });
  __builtin_amdgcn_sched_barrier(0);
  if (has_bias && threadIdx.x < kSmTile) lds_bias[threadIdx.x] = bf16_bits_to_f32(bias_bits);

  // Steps t = 4c + s of K; step t + 1's raw codes are read before step t is decoded and
  // contracted, so the LDS latency hides behind step t's MFMAs; chunk c + 1's wait and barrier
  // come just before its first read.
  using FA = SmFrag<AF, false>;
  using FB = SmFrag<BF, BF == kFp8>;
  uint4 ra[2][FA::kUnits], rb[2][FB::kUnits];
  // this wavefront's copies of chunk c (and the scale bytes before them) have landed; past the
  // barrier, every wavefront's have
  auto chunk_ready = [&](auto cc) {
    constexpr int c = decltype(cc)::value;
    __builtin_amdgcn_s_waitcnt(sm_waitcnt_vm((kSmChunks - 1 - c) * kCp));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  chunk_ready(IntC<0>{});
  fa.template read<0>(ch[0], ra[0]);
  fb.template read<0>(ch[0], rb[0]);
  v16f acc = v16f{};
  static_for<0, 4 * kSmChunks>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    constexpr int c = t / 4, s = t % 4;
    if (c < nch) {
      constexpr int t1 = t + 1, c1 = t1 / 4;
      if constexpr (t1 < 4 * kSmChunks) {
        if (c1 < nch) {
          if constexpr (t1 % 4 == 0) chunk_ready(IntC<c1>{});
          fa.template read<t1 % 4>(ch[c1], ra[t1 & 1]);
          fb.template read<t1 % 4>(ch[c1], rb[t1 & 1]);
        }
      }
      const float sa = fa.template scale<t>(), sb = fb.template scale<t>();
      static_for<0, 4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const bf16x8 av = FA::template decode<q>(ra[t & 1], sa);
        const bf16x8 bv = FB::template decode<q>(rb[t & 1], sb);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, av, acc, 0, 0, 0);
      });
    }
  });
  // copies of chunks past K may still be landing in arrays the epilogue does not use; ch0, which
  // it does use, is past its wait
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  v16f accs[1][1] = {{acc}};
  finish_tile<AF, QUANT, EPI, false, kSmTile, kSmTile, 2, 2>(
      p, accs, [&](int r) { return ch0 + r * (kSmTile * 2); }, lds_bias, has_bias, 0,
      blockIdx.x, m0, n0, bz);
}

template <int AF, int BF, bool BIAS, bool QUANT, int EPI>
hipError_t launch_small(const Args& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_small_kernel<AF, BF, BIAS, QUANT, EPI>), grid, dim3(kSmThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <int AF, int BF>
hipError_t launch_small_formats(const GemmProblem& g, hipStream_t stream) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         (g.M + kSmTile - 1) / kSmTile, (g.N + kSmTile - 1) / kSmTile,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c,
         g.q, g.qs, g.stride_q, g.stride_qs, g.residual, g.stride_res,
         nullptr, nullptr, 1};
  dim3 grid(p.tiles_m * p.tiles_n, g.batch);
  if constexpr (AF == kFp8 || AF == kFp4) {
    if (g.q) {
      if (g.epi == kEpiGelu) return launch_small<AF, BF, true, true, kEpiGelu>(p, grid, stream);
      return g.bias ? launch_small<AF, BF, true, true, kEpiPlain>(p, grid, stream)
                    : launch_small<AF, BF, false, true, kEpiPlain>(p, grid, stream);
    }
  }
  if (g.epi == kEpiResidual) return launch_small<AF, BF, true, false, kEpiResidual>(p, grid, stream);
  if (g.epi == kEpiGelu) return launch_small<AF, BF, true, false, kEpiGelu>(p, grid, stream);
  return g.bias ? launch_small<AF, BF, true, false, kEpiPlain>(p, grid, stream)
                : launch_small<AF, BF, false, false, kEpiPlain>(p, grid, stream);
}

}  // namespace

hipError_t launch_gemm_small(int a_fmt, int b_fmt, const GemmProblem& g, hipStream_t stream) {
  if (!small_kernel_takes(g.K)) return hipErrorInvalidValue;
  if (a_fmt == kFp8 && b_fmt == kFp4) return launch_small_formats<kFp8, kFp4>(g, stream);
  if (a_fmt == kFp8 && b_fmt == kFp8) return launch_small_formats<kFp8, kFp8>(g, stream);
  if (a_fmt == kFp4 && b_fmt == kFp4) return launch_small_formats<kFp4, kFp4>(g, stream);
  if (a_fmt == kBf8 && b_fmt == kFp8Rows) return launch_small_formats<kBf8, kFp8Rows>(g, stream);
  return hipErrorInvalidValue;
}

}  // namespace mx
