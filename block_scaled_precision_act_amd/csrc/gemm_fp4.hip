// Block-scaled GEMM with both operands MXFP4 (E2M1 + per-32 E8M0) for gfx950 at skinny shapes
// (M <= 64) on the scaled f8f6f4 MFMA.  E2M1 values have at most 2 significant bits and span
// under 4 binades, so the products of one scaled MFMA fit its internal adder window and the
// result is the fp32 accumulation of exact products (measured on the device); operands with E4M3
// values, and larger M, go through the bf16-decode path instead.
//
// C[m,n] = bf16_rne(sum_k A[m,k] B[n,k] + bias[n]) with fp32 accumulation on the matrix cores
// ("formats.py" page: decode_fp4 / decode_fp8_block / act_qdq give the decoded operands;
// "AstrAI commit log" page: the bias joins the fp32 sum, which is rounded to bf16 once), or with
// a bf16 residual added, or GELU applied, before that rounding; or that bf16 output quantized to
// MXFP4 for the next A4W4 layer (the "fp4-gemm README" page's GEMM that emits packed FP4).
#include "mx_epilogue.h"
#include "mx_internal.h"
#include "mx_quant.h"

#include <type_traits>

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct Args {
  const uint8_t* a;
  const uint8_t* a_s;
  const uint8_t* b;
  const uint8_t* b_s;
  const uint16_t* bias;
  uint16_t* c;
  int M, N, K;
  int64_t stride_a, stride_as, stride_b, stride_bs, stride_bias, stride_c;
  const uint16_t* res;
  int64_t stride_res;
  uint8_t* q;          // QUANT: packed E2M1 [M, N/2]
  uint8_t* qs;         //        E8M0 [M, N/32]
  int64_t stride_q, stride_qs;
};

__device__ __forceinline__ uint16_t to_bf16(float v) {
  bf16x2 p = {static_cast<__bf16>(v), static_cast<__bf16>(0.0f)};
  return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, p) & 0xFFFFu);
}

// ---------------------------------------------------------------------------------------------
// Skinny MXFP4 x MXFP4 (small M): v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands.
// Operand registers of the 16x16x128 scaled MFMA, as measured on gfx950: lane l holds row
// (l % 16) and K-block g = l / 16 of the 128-wide K step, 16 bytes = 32 E2M1 codes (low nibble
// first) in dwords 0..3, and passes that block's E8M0 byte; accumulator register r of lane l is
// C[4 * (l / 16) + r][l % 16].
// A workgroup owns 16 output columns and all M rows (MT tiles of 16), or half of the row tiles
// (the codes staged through LDS, with room for twice the workgroups in one wave); its W
// wavefronts split the K steps into contiguous ranges and load a group of up to G steps at once
// (one memory round trip per group).  The per-wave partial sums are added in LDS in wave order (deterministic),
// then the bias is added in fp32 and each output is rounded once to bf16.  Rows past M and
// columns past N read zeros through the buffer bound; K blocks past K read zeros through an
// out-of-range offset.
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// After the main loop of either skinny kernel: every wavefront's partial sums go to LDS (`red`,
// [W][MT][NC][64] v4f, free for reuse: every wavefront is past its last operand read), are
// added in wave order (deterministic), the bias is added in fp32 and each output is rounded
// once to bf16; or, QUANT, the bf16 results are quantized to MXFP4 per 32 columns.
template <int MT, int NC, int W, bool BIAS, int EPI, bool QUANT>
__device__ __forceinline__ void skinny_finish(const Args& p, v4f (&acc)[MT][NC], v4f* red, int wave,
                                              int lane, int m0, int n0, int64_t bz) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) red[((wave * MT + t) * NC + c) * 64 + lane] = acc[t][c];
  __syncthreads();
  // Wave w finishes tiles (t, c) = w, w + W, ...: the partial sums are added in wave order.
  // QUANT: the bf16 results go to a [16 MT][32] tile in LDS (over `red`, after a barrier), then
  // each row's 32 values are quantized by the four lanes of a DPP quad.
  uint16_t(*stage)[16 * NC] = reinterpret_cast<uint16_t(*)[16 * NC]>(red);
  v4f sums[(MT * NC + W - 1) / W];
#pragma unroll
  for (int i = 0; i < (MT * NC + W - 1) / W; ++i) {
    const int tc = wave + i * W;
    if (tc < MT * NC) {
      const int t = tc / NC, c = tc % NC;
      v4f sum = red[(t * NC + c) * 64 + lane];
#pragma unroll
      for (int w = 1; w < W; ++w) sum += red[((w * MT + t) * NC + c) * 64 + lane];
      sums[i] = sum;
    }
  }
  if constexpr (QUANT) __syncthreads();      // every wave is done reading `red`
#pragma unroll
  for (int i = 0; i < (MT * NC + W - 1) / W; ++i) {
    const int tc = wave + i * W;
    if (tc >= MT * NC) continue;
    const int t = tc / NC, c = tc % NC;
    const int col = n0 + 16 * c + r16;
    if (!QUANT && col >= p.N) continue;
    float bias = 0.0f;
    if (BIAS && (EPI == kEpiPlain || p.bias != nullptr) && col < p.N)
      bias = bf16_bits_to_f32(p.bias[bz * p.stride_bias + col]);
    uint16_t* out = p.c + bz * p.stride_c;
    const uint16_t* res = p.res + bz * p.stride_res;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lrow = 16 * t + 4 * g + r;       // row within the workgroup's rows
      const int row = m0 + lrow;
      float v = sums[i][r] + bias;
      if constexpr (QUANT) {
        if constexpr (EPI == kEpiGelu) v = gelu_f32(v);
        stage[lrow][16 * c + r16] = to_bf16(v);
      } else {
        if (row >= p.M) continue;
        const int64_t at = static_cast<int64_t>(row) * p.N + col;
        // the residual may be the output itself: this thread reads it before writing it
        if constexpr (EPI == kEpiResidual) v += bf16_bits_to_f32(res[at]);
        if constexpr (EPI == kEpiGelu) v = gelu_f32(v);
        out[at] = to_bf16(v);
      }
    }
  }
  if constexpr (QUANT) {
    static_assert(NC == 2, "a quantized row block needs 32 columns");
    __syncthreads();
    const int idx = threadIdx.x;                // row idx / 4, columns 8 (idx % 4) .. + 8
    if (idx < 16 * MT * 4) {                    // whole quads: the DPP max stays inside
      const int lrow = idx >> 2, ch = idx & 3;
      const int row = m0 + lrow;
      const uint4 v = *reinterpret_cast<const uint4*>(&stage[lrow][8 * ch]);
      const QuantChunkFp4 qc = quant_chunk_fp4(v);
      if (row < p.M) {
        uint8_t* q = p.q + bz * p.stride_q;
        uint8_t* qs = p.qs + bz * p.stride_qs;
        *reinterpret_cast<uint32_t*>(q + static_cast<int64_t>(row) * (p.N / 2) + n0 / 2 + 4 * ch) = qc.codes;
        if (ch == 0) qs[static_cast<int64_t>(row) * (p.N / 32) + n0 / 32] = static_cast<uint8_t>(qc.byte);
      }
    }
  }
}

template <int MT, int NC, int W, int G, bool BIAS, int EPI, bool QUANT>
__global__ __launch_bounds__(64 * W) void gemm_fp4_skinny_kernel(Args p) {
  __shared__ v4f red[W][MT][NC][64];
  const int lane = threadIdx.x & 63;
  // Uniform in the compiler's view too: the per-step buffer offsets derived from it go in
  // scalar registers (no per-lane loop around every load).
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t bz = blockIdx.y;
  const int n0 = blockIdx.x * 16 * NC;
  const int pitch = p.K / 2;
  const int kb_total = p.K / 32;
  const int KT = (p.K + 127) / 128;

  const __amdgpu_buffer_rsrc_t ra = rsrc_of(p.a + bz * p.stride_a, static_cast<uint32_t>(p.M) * pitch);
  const __amdgpu_buffer_rsrc_t ras = rsrc_of(p.a_s + bz * p.stride_as, static_cast<uint32_t>(p.M) * kb_total);
  const __amdgpu_buffer_rsrc_t rb = rsrc_of(p.b + bz * p.stride_b, static_cast<uint32_t>(p.N) * pitch);
  const __amdgpu_buffer_rsrc_t rbs = rsrc_of(p.b_s + bz * p.stride_bs, static_cast<uint32_t>(p.N) * kb_total);

  // Byte offsets at K step 0 (rows past the matrix are clamped to the bound: out of range).
  uint32_t a_off[MT], as_off[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = min(16 * t + r16, p.M);
    a_off[t] = static_cast<uint32_t>(row) * pitch + 16 * g;
    as_off[t] = static_cast<uint32_t>(row) * kb_total + g;
  }
  uint32_t b_off[NC], bs_off[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = min(n0 + 16 * c + r16, p.N);
    b_off[c] = static_cast<uint32_t>(col) * pitch + 16 * g;
    bs_off[c] = static_cast<uint32_t>(col) * kb_total + g;
  }

  const int per = (KT + W - 1) / W;
  const int k_begin = min(wave * per, KT), k_end = min(k_begin + per, KT);

  v4f acc[MT][NC];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[t][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // With K % 128 == 0 a row's scale bytes for the G = 4 steps of a group are 16 consecutive,
  // 4-byte aligned bytes (4 K-blocks per step): one 16-byte load per row fetches them (for a
  // group inside K; the last group of a range may need the one-byte loads), and the
  // lane takes byte 4 s + g of it, a quarter of the load instructions of one byte per lane and
  // step (the loop is bound by the CUs' address-processing rate at the skinny shapes).  A scale
  // byte outside a live step is replaced by 0 (2^-127 times zero codes: nothing), never another
  // row's byte, which could be the E8M0 NaN 0xFF.
  static_assert(G == 4, "16 scale bytes per group");
  const bool vec_scales = (kb_total & 3) == 0;
  for (int k0 = k_begin; k0 < k_end; k0 += G) {
    uint4 av[G][MT], bv[G][NC];
    uint32_t asv[G][MT], bsv[G][NC];
    // every 16-byte row read stays inside that row (rows past M are wholly out of range)
    if (vec_scales && (k0 + G) * 4 <= kb_total) {
      uint4 asq[MT], bsq[NC];
#pragma unroll
      for (int t = 0; t < MT; ++t)
        asq[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               ras, as_off[t] - g, static_cast<uint32_t>(k0) * 4, 0));
#pragma unroll
      for (int c = 0; c < NC; ++c)
        bsq[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rbs, bs_off[c] - g, static_cast<uint32_t>(k0) * 4, 0));
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int kt = k0 + s;
        const bool live = kt < k_end && kt * 4 + g < kb_total;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint32_t d = s == 0 ? asq[t].x : s == 1 ? asq[t].y : s == 2 ? asq[t].z : asq[t].w;
          asv[s][t] = live ? __builtin_amdgcn_ubfe(d, 8 * g, 8) : 0u;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint32_t d = s == 0 ? bsq[c].x : s == 1 ? bsq[c].y : s == 2 ? bsq[c].z : bsq[c].w;
          bsv[s][c] = live ? __builtin_amdgcn_ubfe(d, 8 * g, 8) : 0u;
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int kt = k0 + s;
        const bool live = kt < k_end && kt * 4 + g < kb_total;
        const uint32_t kblk = static_cast<uint32_t>(kt) * 4;
#pragma unroll
        for (int t = 0; t < MT; ++t)
          asv[s][t] = __builtin_amdgcn_raw_buffer_load_b8(ras, live ? as_off[t] : 0x80000000u, kblk, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          bsv[s][c] = __builtin_amdgcn_raw_buffer_load_b8(rbs, live ? bs_off[c] : 0x80000000u, kblk, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const int kt = k0 + s;
      const bool live = kt < k_end && kt * 4 + g < kb_total;
      const uint32_t kbyte = static_cast<uint32_t>(kt) * 64;     // 128 codes = 64 bytes per row
      if (kt < k_end) {         // wave-uniform: a step past the range issues no loads
#pragma unroll
        for (int t = 0; t < MT; ++t)
          av[s][t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   ra, live ? a_off[t] : 0x80000000u, kbyte, 0));
#pragma unroll
        for (int c = 0; c < NC; ++c)
          bv[s][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rb, live ? b_off[c] : 0x80000000u, kbyte, 0));
      } else {
#pragma unroll
        for (int t = 0; t < MT; ++t) av[s][t] = uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < NC; ++c) bv[s][c] = uint4{0u, 0u, 0u, 0u};
      }
    }
    // Straight-line: a step past this wavefront's range has zero codes and zero scale bytes, so
    // its MFMAs add +0 to accumulators that start at +0 and change nothing, and all G steps'
    // loads stay in flight together.
#pragma unroll
    for (int s = 0; s < G; ++s) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        v8i b8 = {static_cast<int>(bv[s][c].x), static_cast<int>(bv[s][c].y),
                  static_cast<int>(bv[s][c].z), static_cast<int>(bv[s][c].w), 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          v8i a8 = {static_cast<int>(av[s][t].x), static_cast<int>(av[s][t].y),
                    static_cast<int>(av[s][t].z), static_cast<int>(av[s][t].w), 0, 0, 0, 0};
          acc[t][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a8, b8, acc[t][c], kFp4, kFp4, 0, static_cast<int>(asv[s][t]), 0,
              static_cast<int>(bsv[s][c]));
        }
      }
    }
  }

  skinny_finish<MT, NC, W, BIAS, EPI, QUANT>(p, acc, &red[0][0][0][0], wave, lane, 0, n0, bz);
}

// The same GEMM with its codes staged through LDS (K % 256 == 0).  A fragment load of the
// 16x16x128 layout reads 16 rows x 64 bytes: 16 half-used 128-byte lines per instruction, and
// at these shapes the kernel is bound by the load instructions' line traffic per CU (measured:
// the same loads over contiguous kilobytes, 8 full lines each, take the load phase from 2.3 to
// 1.5 us at 41x4608x1536).  So each wavefront copies its codes, 2 K steps (128 bytes of a row)
// at a time, straight into its own LDS buffer with full-line copies (copy i of a chunk: rows
// 8 i .. 8 i + 7, lane l the 16 bytes of row 8 i + l / 8 that belong at byte 16 l, the row's
// 16-byte units swizzled by (row / 2) % 8 so that the 16 rows a fragment read takes land in 16
// different bank groups), and reads the fragments from there.  Nothing is shared between
// wavefronts before the epilogue, so no barrier is needed: a wavefront waits for its own copies
// (vmcnt) and then reads.  RING (a range of more than one chunk): chunk c goes to buffer c % 2,
// and the copy of chunk c + 2 leaves once chunk c's fragments are read; otherwise the launch
// gives every wavefront at most one chunk and the kernel has one buffer.  Scale bytes: one 8-byte load per 16-row tile and chunk (the 8
// scale bytes of steps k, k + 1 of the lane's row), issued before the chunk's copies.
template <int MT, int NC, int W, bool RING, bool BIAS, int EPI, bool QUANT>
__global__ __launch_bounds__(64 * W) void gemm_fp4_skinny_lds_kernel(Args p) {
  constexpr int kRows = 16 * (MT + NC);          // a chunk's rows: A tiles, then B tiles
  constexpr int kChunkBytes = kRows * 128;       // 2 K steps of 64 bytes per row
  constexpr int kCopies = kRows / 8;             // 1 KB copies per chunk
  constexpr int kLoads = kCopies + MT + NC;      // vector-memory instructions per chunk
  static_assert(W * MT * NC * 1024 <= W * kChunkBytes, "the reduction fits in buffer 0");
  __shared__ __attribute__((aligned(16))) uint8_t buf0[W * kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[RING ? W * kChunkBytes : 16];
  typedef __attribute__((address_space(3))) void* lds_ptr_t;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t bz = blockIdx.y;
  const int n0 = blockIdx.x * 16 * NC;
  const int m0 = blockIdx.z * 16 * MT;           // the workgroup's rows of A (and C)
  const int pitch = p.K / 2;
  const int kb_total = p.K / 32;
  const int KT = p.K / 128;                      // even: K % 256 == 0

  const __amdgpu_buffer_rsrc_t ra = rsrc_of(p.a + bz * p.stride_a, static_cast<uint32_t>(p.M) * pitch);
  const __amdgpu_buffer_rsrc_t ras = rsrc_of(p.a_s + bz * p.stride_as, static_cast<uint32_t>(p.M) * kb_total);
  const __amdgpu_buffer_rsrc_t rb = rsrc_of(p.b + bz * p.stride_b, static_cast<uint32_t>(p.N) * pitch);
  const __amdgpu_buffer_rsrc_t rbs = rsrc_of(p.b_s + bz * p.stride_bs, static_cast<uint32_t>(p.N) * kb_total);

  // Copy i of a chunk: lane l fetches unit u = (l % 8) ^ swz of row 8 i + l / 8 (of A for
  // i < 2 MT, else of B), the unit that belongs at byte 16 l of the copy's kilobyte.
  uint32_t cp_off[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = 8 * i + (lane >> 3);           // row within the chunk
    const int u = (lane & 7) ^ ((r >> 1) & 7);
    const bool is_a = i < 2 * MT;
    const int row = is_a ? m0 + r : n0 + r - 16 * MT;
    const int lim = is_a ? p.M : p.N;
    cp_off[i] = row < lim ? static_cast<uint32_t>(row) * pitch + 16u * u : 0x80000000u;
  }
  // Scale rows of the lane's tiles (rows past the matrix read zeros).
  uint32_t as_row[MT], bs_row[NC];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = m0 + 16 * t + r16;
    as_row[t] = row < p.M ? static_cast<uint32_t>(row) * kb_total : 0x80000000u;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = n0 + 16 * c + r16;
    bs_row[c] = col < p.N ? static_cast<uint32_t>(col) * kb_total : 0x80000000u;
  }
  // The lane's fragment bytes within a chunk buffer: row 16 t + r16 (A) or 16 (MT + c) + r16
  // (B), unit 4 s + g of step s, swizzled.
  const uint32_t swz = static_cast<uint32_t>((r16 >> 1) & 7);
  const uint32_t frag0 = static_cast<uint32_t>(r16) * 128u;

  // Steps [k_begin, k_end) of K, an even count: whole chunks.
  const int per = ((KT + W - 1) / W + 1) & ~1;
  const int k_begin = min(wave * per, KT), k_end = min(k_begin + per, KT);
  const int nchunks = (k_end - k_begin) / 2;
  const int wbase = wave * kChunkBytes;

  uint2 sa[2][MT], sb[2][NC];                    // scale bytes of a chunk, by buffer
  auto issue = [&](int c, auto par_c) {
    constexpr int PAR = decltype(par_c)::value;
    const int k = k_begin + 2 * c;
#pragma unroll
    for (int t = 0; t < MT; ++t)
      sa[PAR][t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ras, as_row[t], 4 * k, 0));
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
      sb[PAR][c2] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rbs, bs_row[c2], 4 * k, 0));
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      // the buffer named directly (not through a pointer variable), so that the compiler's wait
      // counting tells the copies into one buffer from the reads of the other
      uint8_t* const dst = (PAR ? buf1 : buf0) + wbase + 1024 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(i < 2 * MT ? ra : rb, (lds_ptr_t)dst, 16,
                                               static_cast<int>(cp_off[i]), 64 * k, 0, 0);
    }
  };

  v4f acc[MT][NC];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[t][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto chunk = [&](int c, auto par_c) {
    constexpr int PAR = decltype(par_c)::value;
    // this chunk's loads are done once at most the next chunk's are still in flight
    if (c + 1 < nchunks) __builtin_amdgcn_s_waitcnt((kLoads & 15) | ((kLoads >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
    const uint8_t* const src = (PAR ? buf1 : buf0) + wbase;
    uint4 av[2][MT], bv[2][NC];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t unit = ((4u * s + g) ^ swz) * 16u;
#pragma unroll
      for (int t = 0; t < MT; ++t)
        av[s][t] = *reinterpret_cast<const uint4*>(src + frag0 + 16 * t * 128 + unit);
#pragma unroll
      for (int c2 = 0; c2 < NC; ++c2)
        bv[s][c2] = *reinterpret_cast<const uint4*>(src + frag0 + 16 * (MT + c2) * 128 + unit);
    }
    uint32_t asv[2][MT], bsv[2][NC];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int t = 0; t < MT; ++t) asv[s][t] = __builtin_amdgcn_ubfe(s ? sa[PAR][t].y : sa[PAR][t].x, 8 * g, 8);
#pragma unroll
      for (int c2 = 0; c2 < NC; ++c2) bsv[s][c2] = __builtin_amdgcn_ubfe(s ? sb[PAR][c2].y : sb[PAR][c2].x, 8 * g, 8);
    }
    // every fragment read of this buffer is done before the copy of chunk c + 2 overwrites it
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
    asm volatile("" ::: "memory");
    if (RING && c + 2 < nchunks) issue(c + 2, par_c);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int c2 = 0; c2 < NC; ++c2) {
        const v8i b8 = {static_cast<int>(bv[s][c2].x), static_cast<int>(bv[s][c2].y),
                        static_cast<int>(bv[s][c2].z), static_cast<int>(bv[s][c2].w), 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const v8i a8 = {static_cast<int>(av[s][t].x), static_cast<int>(av[s][t].y),
                          static_cast<int>(av[s][t].z), static_cast<int>(av[s][t].w), 0, 0, 0, 0};
          acc[t][c2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a8, b8, acc[t][c2], kFp4, kFp4, 0, static_cast<int>(asv[s][t]), 0,
              static_cast<int>(bsv[s][c2]));
        }
      }
    }
  };

  if (nchunks > 0) issue(0, std::integral_constant<int, 0>{});
  if (RING && nchunks > 1) issue(1, std::integral_constant<int, 1>{});
  for (int c = 0; c < nchunks; c += 2) {
    chunk(c, std::integral_constant<int, 0>{});
    if (RING && c + 1 < nchunks) chunk(c + 1, std::integral_constant<int, 1>{});
  }
  // every wavefront is past its last operand read (skinny_finish's first barrier precedes any
  // read of `red`, and every copy has landed: the last chunk waited for vmcnt 0)
  __syncthreads();
  skinny_finish<MT, NC, W, BIAS, EPI, QUANT>(p, acc, reinterpret_cast<v4f*>(buf0), wave, lane, m0, n0, bz);
}

template <int MT, int NC, int W, int G>
void launch_unquantized(const GemmProblem& g, dim3 grid, dim3 block, const Args& p,
                        hipStream_t stream) {
  if (g.epi == kEpiResidual)
    hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, true, kEpiResidual, false>), grid,
                       block, 0, stream, p);
  else if (g.epi == kEpiGelu)
    hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, true, kEpiGelu, false>), grid, block,
                       0, stream, p);
  else if (g.bias)
    hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, true, kEpiPlain, false>), grid,
                       block, 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, false, kEpiPlain, false>), grid,
                       block, 0, stream, p);
}

template <int MT, int NC, int W, int G, bool QUANT>
hipError_t launch_skinny(const GemmProblem& g, hipStream_t stream) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c,
         g.residual, g.stride_res, g.q, g.qs, g.stride_q, g.stride_qs};
  dim3 grid((g.N + 16 * NC - 1) / (16 * NC), g.batch);
  const dim3 block(64 * W);
  if constexpr (QUANT) {
    if (g.epi == kEpiGelu)
      hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, true, kEpiGelu, true>), grid, block,
                         0, stream, p);
    else if (g.bias)
      hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, true, kEpiPlain, true>), grid,
                         block, 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_fp4_skinny_kernel<MT, NC, W, G, false, kEpiPlain, true>), grid,
                         block, 0, stream, p);
  } else {
    launch_unquantized<MT, NC, W, G>(g, grid, block, p, stream);
  }
  return hipGetLastError();
}


template <int MT, int NC, int W, bool RING, bool QUANT>
hipError_t launch_skinny_lds(const GemmProblem& g, hipStream_t stream, int mgroups = 1) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c,
         g.residual, g.stride_res, g.q, g.qs, g.stride_q, g.stride_qs};
  const dim3 grid((g.N + 16 * NC - 1) / (16 * NC), g.batch, mgroups);
  const dim3 block(64 * W);
  if constexpr (QUANT) {
    if (g.epi == kEpiGelu)
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, true, kEpiGelu, true>), grid, block,
                         0, stream, p);
    else if (g.bias)
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, true, kEpiPlain, true>), grid,
                         block, 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, false, kEpiPlain, true>), grid,
                         block, 0, stream, p);
  } else {
    if (g.epi == kEpiResidual)
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, true, kEpiResidual, false>), grid,
                         block, 0, stream, p);
    else if (g.epi == kEpiGelu)
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, true, kEpiGelu, false>), grid,
                         block, 0, stream, p);
    else if (g.bias)
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, true, kEpiPlain, false>), grid,
                         block, 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_fp4_skinny_lds_kernel<MT, NC, W, RING, false, kEpiPlain, false>), grid,
                         block, 0, stream, p);
  }
  return hipGetLastError();
}

// The LDS kernel with 16-column workgroups of MT row tiles each and `mgroups` workgroups per
// column block (row tiles [MT i, MT i + MT) in workgroup i).
template <int MT>
hipError_t launch_skinny_lds_rows(const GemmProblem& g, int mgroups, hipStream_t stream) {
  const int kt = (g.K + 127) / 128;
  if (kt <= 8) return launch_skinny_lds<MT, 1, 4, false, false>(g, stream, mgroups);
  if (kt <= 12) return launch_skinny_lds<MT, 1, 6, false, false>(g, stream, mgroups);
  if constexpr (MT + 1 <= 4) return launch_skinny_lds<MT, 1, 8, true, false>(g, stream, mgroups);
  return launch_skinny_lds<MT, 1, 4, true, false>(g, stream, mgroups);
}

template <int MT>
hipError_t launch_skinny_mt(const GemmProblem& g, int cus, hipStream_t stream) {
  const int kt = (g.K + 127) / 128;
  if (g.K % 256 == 0) {
    // Codes staged through LDS.  Wavefronts: one chunk of 2 steps each for up to 12 steps of K (4 or 6 wavefronts, one
    // chunk buffer), else 8 with a ring of two buffers where those fit in 128 KB of LDS
    // (16 (MT + NC) rows x 128 bytes each), else 4.
    // 32 columns per workgroup where 16-column workgroups would not fit in one wave of the CUs:
    // a CU then copies A's rows once for 32 columns instead of once per 16 (a CU running two
    // 16-column workgroups copies them twice).
    const int64_t wg16 = static_cast<int64_t>((g.N + 15) / 16) * g.batch;
    // Where even twice the 16-column grid fits in one wave, two workgroups per column block,
    // each with half the row tiles: a CU copies half of A's rows (plus the block's B rows).
    if constexpr (MT >= 2) {
      if (!g.q && 2 * wg16 <= cus) return launch_skinny_lds_rows<(MT + 1) / 2>(g, 2, stream);
    }
    if (g.q || wg16 > cus) {
      if (g.q) {
        if (kt <= 8) return launch_skinny_lds<MT, 2, 4, false, true>(g, stream);
        if (kt <= 12) return launch_skinny_lds<MT, 2, 6, false, true>(g, stream);
        if constexpr (MT + 2 <= 4) return launch_skinny_lds<MT, 2, 8, true, true>(g, stream);
        return launch_skinny_lds<MT, 2, 4, true, true>(g, stream);
      }
      if (kt <= 8) return launch_skinny_lds<MT, 2, 4, false, false>(g, stream);
      if (kt <= 12) return launch_skinny_lds<MT, 2, 6, false, false>(g, stream);
      if constexpr (MT + 2 <= 4) return launch_skinny_lds<MT, 2, 8, true, false>(g, stream);
      return launch_skinny_lds<MT, 2, 4, true, false>(g, stream);
    }
    return launch_skinny_lds_rows<MT>(g, 1, stream);
  }
  if (g.q) {   // quantized output: 32 columns per workgroup (one scale block of each row)
    if (kt >= 32) return launch_skinny<MT, 2, 8, 4, true>(g, stream);
    return launch_skinny<MT, 2, 4, 4, true>(g, stream);
  }
  if (kt >= 32) return launch_skinny<MT, 1, 8, 4, false>(g, stream);   // long K: 8 wavefronts
  return launch_skinny<MT, 1, 4, 4, false>(g, stream);
}

}  // namespace

hipError_t launch_gemm_fp4_mfma(const GemmProblem& p, int cus, hipStream_t stream) {
  // Skinny problems only (M <= 64): 16- or 32-column workgroups with split K.
  if (p.M <= 16) return launch_skinny_mt<1>(p, cus, stream);
  if (p.M <= 32) return launch_skinny_mt<2>(p, cus, stream);
  if (p.M <= 48) return launch_skinny_mt<3>(p, cus, stream);
  return launch_skinny_mt<4>(p, cus, stream);
}

hipError_t launch_gemm(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                       hipStream_t stream) {
  // Both operands MXFP4: the scaled FP4 MFMA for the skinny (decode-like) shapes, M <= 64; from
  // M = 65 on, the tiled bf16-decode kernel (3.7x faster at 4096x7168x2048 than one wavefront
  // per 32x32 tile of the scaled FP4 MFMA, as first built here).
  if (a_fmt == kFp4 && b_fmt == kFp4 && p.M <= 64)
    return launch_gemm_fp4_mfma(p, dev.cu_count > 0 ? dev.cu_count : 256, stream);
  return launch_gemm_bf16(a_fmt, b_fmt, p, dev, stream);
}

}  // namespace mx
