// Block-scaled GEMM with FP8 operands for gfx950: decode to exact bf16, contract on the bf16
// MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation, fused fp32 bias, one bf16 rounding.
//
// What is computed ("formats.py" page: decode_fp4 / decode_fp8_block / act_qdq; "AstrAI commit
// log" page: the bias joins the fp32 sum, which is then rounded to bf16 once):
//   C[m,n] = bf16_rne( sum_k A[m,k] B[n,k] + bias[n] ),  A, B the exactly decoded operands.
//
// Why bf16 and not the scaled FP8 MFMA: on gfx950 the FP8 (E4M3) matrix instructions align the
// products of one instruction to a narrow fixed-point window before adding them, so products far
// below the largest one lose low bits (about 2^-13 of the largest product per instruction, measured
// on the device).  That breaks the 2^-20 * sum|a*b| accuracy this GEMM promises on a few outputs
// per thousand.  A decoded operand value is a 4-bit (E4M3) or 2-bit (E2M1) significand times a
// power of two, so with its E8M0 scale folded in it is EXACTLY a bf16 value; the bf16 MFMA forms
// exact products and accumulates them in fp32, which meets the bound.
//
// Design (per workgroup of WM x WN wavefronts, tile BM x BN, K step 64):
//   * A is decoded once per workgroup: 16-byte global loads of raw codes and the E8M0 byte of their
//     32-block go to registers one K step ahead, v_cvt_scalef32_pk_bf16_{fp8,fp4} decode two values
//     per instruction with the scale folded in, and the bf16 rows (128 B, 16-byte chunks swizzled
//     by row) are written to an LDS stage;
//   * B stays raw in LDS (E4M3 or packed E2M1, 64 or 32 bytes per row and K step): every wavefront
//     reads the raw codes of its own B rows and decodes them in registers.  LDS writes cost about
//     2.5x what LDS reads cost per byte on gfx950, so staging B raw (1 or 0.5 byte per value instead
//     of 2) saves more than the decode work it repeats in the WM wavefronts that share a B row;
//   * K order inside a step: the MFMA's lane group h of sub-step s takes K [32h + 8s, 32h + 8s + 8)
//     of the step (the same permutation for A and B, so the sum is unchanged).  A lane's four
//     sub-steps then cover one whole 32-block of its row: one 16- or 32-byte raw read and one scale
//     per B row and step;
//   * two LDS stages; the next stage is written in the first three sub-steps, a barrier follows,
//     and the last sub-step's MFMAs hide the first reads of the next stage;
//   * wavefront tile (BM/WM) x (BN/WN) of 32x32 MFMA blocks held in accumulator registers;
//   * the workgroup -> tile map keeps consecutive tiles on one XCD (workgroups are dealt to the 8
//     XCDs round-robin) and walks them in groups of kGroupM tile rows, so an XCD's L2 holds the
//     A rows and B rows its running tiles share;
//   * epilogue: fp32 + bias (+ a bf16 residual, or GELU), one RNE rounding, staged through LDS
//     for 16-byte row stores; or, for the quantizing entry points, the same bf16 tile quantized
//     per 32 columns to E4M3 + E8M0 (the next layer's activation operand) without writing the
//     bf16 values out.
#include <atomic>

#include "gemm_common.h"

namespace mx {
namespace {

constexpr int kBK = 64;          // K elements per stage
constexpr int kRowBytes = 128;   // one decoded LDS row: 64 bf16
constexpr int kParts = 3;        // sub-steps that stage the next K step (the fourth holds the barrier)
// Decoded rows are 128 B (64 bf16 = 8 chunks of 16 B).  Chunk c of row r is stored at chunk
// c ^ swz(r), swz(r) = (r & 7) ^ parity(bits 1..3 of r), period 16 in r.  It keeps every LDS pass
// free of bank conflicts, whether a pass serves 8 lanes (128 B of banks) or 16 lanes (256 B), for
// the fragment reads (8 or 16 consecutive rows at one logical chunk), the FP8 decode writes (rows
// r, r+1 x 4 pieces of 2 chunks) and the FP4 decode writes (rows r..r+3 x 2 pieces of 4 chunks).
// Found by exhaustive search over period-16 tables.
__device__ __forceinline__ int swz(int row) {
  return (row & 7) ^ (__builtin_popcount((row >> 1) & 7) & 1);
}

__device__ __forceinline__ uint32_t lds_offset(int row, int chunk) {
  return static_cast<uint32_t>(row * kRowBytes + ((chunk ^ swz(row)) << 4));
}

// Raw code rows hold one K step of one operand row (E4M3: 64 B = 4 units of 16 B; E2M1: 32 B =
// 2 units).  Unit u of row r is stored at u ^ graw(r).  16 consecutive rows reading one logical
// unit, and the staging writes (4 rows x 4 units or 8 rows x 2 units per 16 lanes), then touch
// 16 distinct 16-byte bank groups.  Period 16 in r.
template <int FMT>
__device__ __forceinline__ int graw(int row) {
  return byte_codes(FMT) ? (row >> 2) & 3 : (row >> 3) & 1;
}

// Moves one operand's codes for one K step from global memory into an LDS stage region.
// A row of one K step is FP8: 4 pieces of 16 codes; FP4: 2 pieces of 32 codes (16 bytes each).
// Thread t owns pieces c = t + i*NT (i < kPer): row c / kPieces, piece c % kPieces.  Rows past
// the matrix and the K half past the end of a partial last step read zeros through the buffer
// bound; the per-step advance is a scalar offset.
// DECODE: each piece is decoded with its E8M0 scale into bf16 chunks of 128-byte rows; otherwise
// the raw 16 bytes are stored into rows of kStepBytes.
// Piece i is staged in part PART0 + i * NPART / kPer of a K step and reloaded right after, for
// the step after next, so every piece has a whole K step to arrive with a single register set.
template <int FMT, int ROWS, int NT, bool DECODE, int PART0, int NPART>
struct Stager {
  static constexpr int kPieces = byte_codes(FMT) ? 4 : 2;
  static constexpr int kStepBytes = byte_codes(FMT) ? 64 : 32;   // bytes of a row per K step
  static constexpr int kTotal = ROWS * kPieces;
  static constexpr int kPer = (kTotal + NT - 1) / NT;
  static constexpr bool kAll = kTotal % NT == 0;
  static constexpr int kRowStride = NT / kPieces;                // rows between pieces i, i+1
  static constexpr int kChunksPerPiece = DECODE ? (byte_codes(FMT) ? 2 : 4) : 1;
  static constexpr int kChunks = kPer * kChunksPerPiece;
  static constexpr uint32_t kOob = 0x80000000u;                  // past any buffer bound
  static_assert(NT % kPieces == 0 && kRowStride % 16 == 0, "swizzle period");
  static_assert(PART0 >= 0 && PART0 + NPART <= kParts && NPART >= 1, "parts");

  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t voff[kPer];      // byte offset of piece i at K step 0
  uint32_t soff[kPer];      // byte offset of its scale byte at K step 0
  uint32_t lds0;            // LDS offset (stage-relative) of piece 0
  bool upper;               // the thread's pieces cover K [32, 64) of a step
  uint4 raw[kPer];
  uint32_t sbyte[kPer];

  __device__ __forceinline__ void init(const uint8_t* base, const uint8_t* sbase, int row0,
                                       int rows_valid, int K, bool block_scales, uint32_t region) {
    const int pitch = byte_codes(FMT) ? K : K / 2;
    const int kb_total = K / 32;
    const int t = threadIdx.x;
    const int p = t % kPieces;
    const int koff = (byte_codes(FMT) ? 16 : 32) * p;
    upper = koff >= 32;
    const int srows = block_scales ? (rows_valid + 31) / 32 : rows_valid;
    codes = make_rsrc(base, static_cast<uint32_t>(rows_valid) * static_cast<uint32_t>(pitch));
    if (DECODE)
      scales = make_rsrc(sbase, static_cast<uint32_t>(srows) * static_cast<uint32_t>(kb_total));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = min(row0 + t / kPieces + i * kRowStride, rows_valid);   // == rows_valid: OOB
      voff[i] = static_cast<uint32_t>(r) * pitch + 16 * p;
      const int sr = block_scales ? r / 32 : r;
      soff[i] = static_cast<uint32_t>(sr) * kb_total + koff / 32;
    }
    const int lrow = t / kPieces;
    if (DECODE)
      lds0 = region + lds_offset(lrow, kChunksPerPiece * p);
    else
      lds0 = region + static_cast<uint32_t>(lrow * kStepBytes + ((p ^ graw<FMT>(lrow)) << 4));
  }

  // Loads piece I of K step kt; `partial` marks a last step holding only 32 valid K.
  template <int I>
  __device__ __forceinline__ void load_piece(int kt, bool partial) {
    const uint32_t v = (partial && upper) ? kOob : voff[I];
    raw[I] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(codes, v, kt * kStepBytes, 0));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DECODE) {
      // the scale byte of a 32-block past K (upper half of a last half step) is not read
      sbyte[I] = __builtin_amdgcn_raw_buffer_load_b8(scales, (partial && upper) ? kOob : soff[I],
                                                     kt * 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ void load_all(int kt, bool partial) {
    static_for<0, kPer>([&](auto ic) { load_piece<decltype(ic)::value>(kt, partial); });
  }

  static constexpr int piece_part(int i) { return PART0 + (i * NPART) / kPer; }
  static constexpr int part_of(int q) { return piece_part(q / kChunksPerPiece); }

  // Writes chunk Q (decoded, or the raw piece) to the LDS stage.  The chunks of one decoded piece
  // are consecutive logical chunks of one row: the physical chunk of logical (base + j) is
  // (base ^ swz) ^ j because base is a multiple of kChunksPerPiece.  Rows i * kRowStride apart
  // share the swizzle (period 16).
  template <int Q>
  __device__ __forceinline__ void store_chunk(uint8_t* stage) const {
    constexpr int i = Q / kChunksPerPiece, j = Q % kChunksPerPiece;
    if (!kAll && !(static_cast<int>(threadIdx.x) + i * NT < kTotal)) return;
    if constexpr (!DECODE) {
      *reinterpret_cast<uint4*>(stage + lds0 + i * kRowStride * kStepBytes) = raw[i];
    } else {
      const float s = e8m0_value(sbyte[i]);
      const uint32_t c0 = (lds0 >> 4) & 7;
      uint8_t* dst = stage + (lds0 - (c0 << 4)) + i * kRowStride * kRowBytes + ((c0 ^ j) << 4);
      uint4 o;
      if constexpr (FMT == kBf8) {
        o = j == 0 ? decode_bf8_pair(raw[i].x, raw[i].y, s) : decode_bf8_pair(raw[i].z, raw[i].w, s);
      } else if constexpr (byte_codes(FMT)) {
        o = j == 0 ? decode_fp8_pair(raw[i].x, raw[i].y, s) : decode_fp8_pair(raw[i].z, raw[i].w, s);
      } else {
        const uint32_t d = j == 0 ? raw[i].x : j == 1 ? raw[i].y : j == 2 ? raw[i].z : raw[i].w;
        o = decode_fp4_dword(d, s);
      }
      *reinterpret_cast<uint4*>(dst) = o;
    }
  }

  template <int PART>
  static constexpr int chunks_in_part() {
    int n = 0;
    for (int q = 0; q < kChunks; ++q) n += part_of(q) == PART ? 1 : 0;
    return n;
  }

  // Index of the N-th chunk staged in part PART.
  template <int PART, int N>
  static constexpr int nth_chunk() {
    int n = 0;
    for (int q = 0; q < kChunks; ++q) {
      if (part_of(q) == PART) {
        if (n == N) return q;
        ++n;
      }
    }
    return -1;
  }

  // The reloads after part PART: every piece staged in that part, in a fixed order (each load is
  // fenced from the scheduler), so every path into the K loop, prologue included, leaves the same
  // sequence of outstanding loads and the waits the loop needs stay as shallow as the data allow.
  template <int PART>
  __device__ __forceinline__ void load_part(int kt, bool partial) {
    static_for<0, kPer>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (piece_part(i) == PART) load_piece<i>(kt, partial);
    });
  }

  __device__ __forceinline__ void store_all(uint8_t* stage) const {
    static_for<0, kChunks>([&](auto qc) { store_chunk<decltype(qc)::value>(stage); });
  }
};

// The B operand of one wavefront: TN tiles of 32 rows.  Each step, lane (row l % 32, group h)
// reads the raw codes of K [32h, 32h+32) of its row from the LDS stage (E4M3: 32 bytes, E2M1: 16
// bytes) and its E8M0 byte (loaded from global memory one step ahead), and decodes the 8 values of
// each sub-step into the MFMA's bf16 operand just before they are needed.
template <int BF, int TN>
struct BRegs {
  static constexpr int kQ = byte_codes(BF) ? 2 : 1;        // 16-byte units per row per lane
  static constexpr int kPitch = byte_codes(BF) ? 64 : 32;  // raw row bytes per step
  uint4 raw[TN][kQ];
  float scale[TN];
  uint32_t sbyte[TN];           // scale bytes of the step loaded next
  __amdgpu_buffer_rsrc_t srsrc;
  uint32_t soff[TN];
  uint32_t lds_off[kQ];         // stage-relative LDS offset of tile 0

  __device__ __forceinline__ void init(const uint8_t* sbase, int n_first, int N, int K,
                                       uint32_t region, int row_local) {
    const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int kb_total = K / 32;
    const int srows = BF == kFp8 ? (N + 31) / 32 : N;    // 32x32 blocks, or per row
    srsrc = make_rsrc(sbase, static_cast<uint32_t>(srows) * static_cast<uint32_t>(kb_total));
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n_first + 32 * j + l32;
      const int sr = min(BF == kFp8 ? n / 32 : n, srows);               // == srows: OOB -> 0
      soff[j] = static_cast<uint32_t>(sr) * kb_total + h;
    }
    const int r = row_local + l32;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = byte_codes(BF) ? 2 * h + q : h;
      lds_off[q] = region + static_cast<uint32_t>(r * kPitch + ((u ^ graw<BF>(r)) << 4));
    }
  }

  // Scale bytes of step kt; `partial`: a last half step, whose second 32-block (lane group 1)
  // is past K and is not read.
  __device__ __forceinline__ void load_scales(int kt, bool partial) {
    const bool skip = partial && (threadIdx.x & 32) != 0;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sbyte[j] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, skip ? 0x80000000u : soff[j], kt * 2, 0);
  }

  __device__ __forceinline__ void take_scales() {
#pragma unroll
    for (int j = 0; j < TN; ++j) scale[j] = e8m0_value(sbyte[j]);
  }

  template <int J, int Q>
  __device__ __forceinline__ void read_raw(const uint8_t* stage) {
    raw[J][Q] = *reinterpret_cast<const uint4*>(stage + lds_off[Q] + 32 * J * kPitch);
  }

  __device__ __forceinline__ void read_raw_all(const uint8_t* stage) {
    static_for<0, TN * kQ>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      read_raw<t / kQ, t % kQ>(stage);
    });
  }

  // bf16 operand of tile J for sub-step S: K [32h + 8S, 32h + 8S + 8) of the row.
  template <int S, int J>
  __device__ __forceinline__ void decode(bf16x8& out) const {
    uint4 o;
    if constexpr (byte_codes(BF)) {
      const uint4 q = raw[J][S >> 1];
      o = (S & 1) ? decode_fp8_pair(q.z, q.w, scale[J]) : decode_fp8_pair(q.x, q.y, scale[J]);
    } else {
      const uint32_t d = S == 0 ? raw[J][0].x : S == 1 ? raw[J][0].y : S == 2 ? raw[J][0].z : raw[J][0].w;
      o = decode_fp4_dword(d, scale[J]);
    }
    out = __builtin_bit_cast(bf16x8, o);
  }

  template <int S>
  __device__ __forceinline__ void decode_all(bf16x8 (&out)[TN]) const {
    static_for<0, TN>([&](auto jc) { decode<S, decltype(jc)::value>(out[decltype(jc)::value]); });
  }
};

template <int TM>
__device__ __forceinline__ void read_a(const uint8_t* stage, uint32_t a_base, uint32_t coff,
                                       bf16x8 (&f)[TM]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
    f[i] = *reinterpret_cast<const bf16x8*>(stage + a_base + i * 32 * kRowBytes + coff);
}

// One K step on LDS stage `cur`, as four sub-steps of TM x TN MFMAs.  MORE: stage the next step
// into `nxt` during sub-steps 0..2, then (after a barrier) read its first operands during
// sub-step 3; RELOAD: reload the staged pieces for step kt_load.  On entry fa[0] / fb[0] hold
// sub-step 0's operands; on exit (MORE) they hold the next step's.
// The other work of a sub-step is cut into tasks (an A fragment read, a raw B read, a B tile
// decode, one staged chunk) that are spread evenly over the slots after its MFMAs; each slot is
// fenced from the scheduler so the matrix pipe gets an MFMA between every few other instructions.
template <bool MORE, bool RELOAD, int FA, int TM, int TN, class SA, class SB, class BR>
__device__ __forceinline__ void k_step(const uint8_t* cur, uint8_t* nxt, uint32_t a_base,
                                       const uint32_t (&coff)[4], SA& sa, SB& sb, BR& br,
                                       bf16x8 (&fa)[FA][TM], bf16x8 (&fb)[2][TN],
                                       v16f (&acc)[TM][TN], int kt_load, bool partial_load) {
  static_for<0, 4>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int nb = (s + 1) & 1;                                      // operand buffer filled
    constexpr bool last = s == 3;
    constexpr int kRaw = (last && MORE) ? TN * BR::kQ : 0;               // raw B reads of nxt
    // A fragment reads: one sub-step ahead, or (FA == 4) all four sub-steps of the next K step
    // after the barrier, so a wavefront with one MFMA per sub-step waits for LDS once per step.
    constexpr bool kAllRead = FA == 4;
    constexpr int kRd = kAllRead ? ((last && MORE) ? 4 * TM : 0) : ((!last || MORE) ? TM : 0);
    constexpr int kDec = (!last || MORE) ? TN : 0;                        // B tile decodes
    constexpr int kA = (!last && MORE) ? SA::template chunks_in_part<s>() : 0;
    constexpr int kB = (!last && MORE) ? SB::template chunks_in_part<s>() : 0;
    constexpr int kTasks = kRaw + kRd + kDec + kA + kB;
    constexpr int kM = TM * TN;
    if constexpr (last && MORE) {
      // Every write to `nxt` and every read of `cur` is complete in every wavefront past here.
      __syncthreads();
      br.take_scales();
    }
    auto task = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if constexpr (t < kRaw) {
        br.template read_raw<t / BR::kQ, t % BR::kQ>(nxt);
      } else if constexpr (t < kRaw + kRd && kAllRead) {
        constexpr int sub = (t - kRaw) / TM, i = (t - kRaw) % TM;
        fa[sub][i] = *reinterpret_cast<const bf16x8*>(nxt + a_base + i * 32 * kRowBytes + coff[sub]);
      } else if constexpr (t < kRaw + kRd) {
        constexpr int i = t - kRaw;
        const uint8_t* stage = last ? nxt : cur;
        fa[nb][i] = *reinterpret_cast<const bf16x8*>(stage + a_base + i * 32 * kRowBytes +
                                                     coff[(s + 1) & 3]);
      } else if constexpr (t < kRaw + kRd + kDec) {
        constexpr int j = t - kRaw - kRd;
        br.template decode<(s + 1) & 3, j>(fb[nb][j]);
      } else if constexpr (t < kRaw + kRd + kDec + kA) {
        sa.template store_chunk<SA::template nth_chunk<s, t - kRaw - kRd - kDec>()>(nxt);
      } else {
        sb.template store_chunk<SB::template nth_chunk<s, t - kRaw - kRd - kDec - kA>()>(nxt);
      }
    };
    static_for<0, kM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int i = m / TN, j = m % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s & 1][j], fa[kAllRead ? s : s & 1][i],
                                                          acc[i][j], 0, 0, 0);
      static_for<m * kTasks / kM, (m + 1) * kTasks / kM>(task);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (RELOAD && !last) {
      sa.template load_part<s>(kt_load, partial_load);
      sb.template load_part<s>(kt_load, partial_load);
    }
  });
}

// QUANT: instead of the bf16 output, write its per-32 codes and E8M0 bytes (the next layer's
// activation operand), computed from the same bf16 values with the producers' arithmetic: E4M3
// (act_quant) when A is E4M3, packed E2M1 (the MXFP4 producer) when A is E2M1, so an A4W4 layer
// feeds the next A4W4 layer.  QUANT combines with kEpiGelu (GELU before the bf16 rounding).
// EPI (bf16 output only): kEpiResidual adds the bf16 residual [M, N] before the rounding,
// kEpiGelu applies GELU to (sum + bias); both take the bias pointer as optional (BIAS is true
// for them and a null bias adds nothing).
// SPLIT (splits == 2): workgroup b computes K range (b % 2) of tile b / 2; the first of the two to
// finish publishes its fp32 partial tile, the second adds it to its own and runs the epilogue
// (finish_tile).
// LDS of one workgroup: the two operand stages, reused by the bf16 output tile of the epilogue,
// then the tile's bias as fp32.
template <int AF, int BF, int BM, int BN>
constexpr int lds_tile_bytes() {
  constexpr int stages = 2 * (BM * kRowBytes + BN * (byte_codes(BF) ? 64 : 32));
  constexpr int tile = BM * BN * 2;
  return stages > tile ? stages : tile;
}

template <int AF, int BF, int BM, int BN>
constexpr int lds_bytes() {
  return lds_tile_bytes<AF, BF, BM, BN>() + BN * 4;
}

template <int AF, int BF, bool BIAS, bool QUANT, int EPI, bool SPLIT, int BM, int BN, int WM,
          int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(Args p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;     // WM x WN wavefronts
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  constexpr int kBPitch = byte_codes(BF) ? 64 : 32;
  constexpr int kBRegion = BM * kRowBytes;
  constexpr int kStageBytes = kBRegion + BN * kBPitch;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;

  int tile_id = blockIdx.x, ntiles = gridDim.x, split = 0;
  if constexpr (SPLIT) {
    split = blockIdx.x % p.splits;
    tile_id = blockIdx.x / p.splits;
    ntiles = gridDim.x / p.splits;
  }
  int tm, tn;
  tile_of(tile_id, ntiles, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t bz = blockIdx.y;
  const int m0 = tm * BM, n0 = tn * BN;

  constexpr int kPerA = Stager<AF, BM, NT, true, 0, 1>::kPer;
  constexpr int kPerB = Stager<BF, BN, NT, false, 0, 1>::kPer;
  constexpr int kNA = kPerA < 2 ? kPerA : 2;
  constexpr int kNB = kPerB < 2 ? kPerB : 2;
  Stager<AF, BM, NT, true, 0, kNA> sa;
  Stager<BF, BN, NT, false, kParts - kNB, kNB> sb;
  sa.init(p.a + bz * p.stride_a, p.a_s + bz * p.stride_as, m0, p.M, p.K, false, 0);
  sb.init(p.b + bz * p.stride_b, nullptr, n0, p.N, p.K, BF == kFp8, kBRegion);
  BRegs<BF, TN> br;
  br.init(p.b_s + bz * p.stride_bs, n0 + wn * WTN, p.N, p.K, kBRegion, wn * WTN);

  // A fragment rows wm*WTM + 32i + l32 share swz(l32), so four chunk offsets (one per sub-step,
  // chunk 4h + s: K [32h + 8s, 32h + 8s + 8)) serve every fragment.
  const uint32_t a_base = static_cast<uint32_t>((wm * WTM + l32) * kRowBytes);
  uint32_t coff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) coff[ks] = static_cast<uint32_t>(((4 * h + ks) ^ swz(l32)) << 4);

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
  // One 32x32 block per wavefront: its four sub-steps' A fragments are read together.
  constexpr int kFa = TM * TN == 1 ? 4 : 2;
  bf16x8 fa[kFa][TM], fb[2][TN];

  // The tile's bias as fp32 in LDS for the epilogue: thread c loads column c here, with the
  // first step's operand loads behind it, and stores it to LDS just before the prologue's
  // barrier, so its latency is hidden behind theirs.
  static_assert(BN <= NT, "one bias value per thread");
  float* const lds_bias = reinterpret_cast<float*>(lds + lds_tile_bytes<AF, BF, BM, BN>());
  const bool has_bias = BIAS && (EPI == kEpiPlain || p.bias != nullptr);
  uint32_t bias_bits = 0;        // raw, so that nothing waits for the load before the store
  if (has_bias)
    bias_bits = p.bias[bz * p.stride_bias +
                       min(n0 + min(static_cast<int>(threadIdx.x), BN - 1), p.N - 1)];

  // Pipeline: step k's codes are staged into LDS stage k & 1 during step k-1, piece by piece, and
  // each piece is reloaded for step k+1 right after it is staged.  Steps [k0, k0 + KT) of the
  // KT_all steps of K (all of them unless SPLIT); loads take absolute step indices.
  const int KT_all = (p.K + kBK - 1) / kBK;
  int k0 = 0, KT = KT_all;
  if constexpr (SPLIT) {
    k0 = static_cast<int>(static_cast<int64_t>(split) * KT_all / p.splits);
    KT = static_cast<int>(static_cast<int64_t>(split + 1) * KT_all / p.splits) - k0;
  }
  const int last_partial = (p.K % kBK) != 0 ? KT_all - 1 : -1;
  sa.load_all(k0, last_partial == k0);
  sb.load_all(k0, last_partial == k0);
  br.load_scales(k0, last_partial == k0);
  sa.store_all(lds);
  sb.store_all(lds);
  if (KT > 1) {
    static_for<0, kParts>([&](auto pc) {
      constexpr int P = decltype(pc)::value;
      sa.template load_part<P>(k0 + 1, last_partial == k0 + 1);
      sb.template load_part<P>(k0 + 1, last_partial == k0 + 1);
    });
  }
  if (has_bias && static_cast<int>(threadIdx.x) < BN)
    lds_bias[threadIdx.x] = bf16_bits_to_f32(bias_bits);
  __syncthreads();
  br.take_scales();
  static_for<0, kFa == 4 ? 4 : 1>([&](auto kc) {
    constexpr int ks = decltype(kc)::value;
    read_a<TM>(lds, a_base, coff[ks], fa[ks]);
  });
  br.read_raw_all(lds);
  br.template decode_all<0>(fb[0]);
  if (KT > 1) br.load_scales(k0 + 1, last_partial == k0 + 1);

  int kt = 0;
  for (; kt + 2 < KT; ++kt) {
    k_step<true, true>(lds + (kt & 1) * kStageBytes, lds + ((kt + 1) & 1) * kStageBytes, a_base,
                       coff, sa, sb, br, fa, fb, acc, k0 + kt + 2, k0 + kt + 2 == last_partial);
    br.load_scales(k0 + kt + 2, last_partial == k0 + kt + 2);
  }
  if (kt + 1 < KT) {
    k_step<true, false>(lds + (kt & 1) * kStageBytes, lds + ((kt + 1) & 1) * kStageBytes, a_base,
                        coff, sa, sb, br, fa, fb, acc, 0, false);
    ++kt;
  }
  k_step<false, false>(lds + (kt & 1) * kStageBytes, lds, a_base, coff, sa, sb, br, fa, fb, acc,
                       0, false);

  finish_tile<AF, QUANT, EPI, SPLIT, BM, BN, WM, WN>(
      p, acc, [&](int r) { return lds + r * (BN * 2); }, lds_bias, has_bias, split, tile_id, m0, n0,
      bz);
}


template <int AF, int BF, bool BIAS, bool QUANT, int EPI, int BM, int BN, int WM, int WN,
          bool SPLIT = false>
hipError_t launch_kernel(const Args& p, dim3 grid, int device, hipStream_t stream) {
  constexpr int kLds = lds_bytes<AF, BF, BM, BN>();
  static_assert(kLds + 16 <= 160 * 1024, "LDS");
  auto k = gemm_bf16_kernel<AF, BF, BIAS, QUANT, EPI, SPLIT, BM, BN, WM, WN>;
  // The dynamic-LDS limit (above 64 KB needs the attribute) is raised once per kernel and device
  // (device ids are below 64); two threads that race here both set the same value.
  static std::atomic<uint64_t> raised{0};
  const uint64_t bit = uint64_t{1} << (device & 63);
  if ((raised.load(std::memory_order_acquire) & bit) == 0) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(k, grid, dim3(64 * WM * WN), kLds, stream, p);
  return hipGetLastError();
}

template <int AF, int BF, int BM, int BN, int WM, int WN>
hipError_t launch_tile(const GemmProblem& g, int device, hipStream_t stream) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         (g.M + BM - 1) / BM, (g.N + BN - 1) / BN,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c,
         g.q, g.qs, g.stride_q, g.stride_qs, g.residual, g.stride_res,
         nullptr, nullptr, 1};
  dim3 grid(p.tiles_m * p.tiles_n, g.batch);
  if constexpr (AF == kFp8 || AF == kFp4) {
    if (g.q) {
      if (g.epi == kEpiGelu)
        return launch_kernel<AF, BF, true, true, kEpiGelu, BM, BN, WM, WN>(p, grid, device, stream);
      return g.bias ? launch_kernel<AF, BF, true, true, kEpiPlain, BM, BN, WM, WN>(p, grid, device, stream)
                    : launch_kernel<AF, BF, false, true, kEpiPlain, BM, BN, WM, WN>(p, grid, device, stream);
    }
  }
  if (g.epi == kEpiResidual)
    return launch_kernel<AF, BF, true, false, kEpiResidual, BM, BN, WM, WN>(p, grid, device, stream);
  if (g.epi == kEpiGelu)
    return launch_kernel<AF, BF, true, false, kEpiGelu, BM, BN, WM, WN>(p, grid, device, stream);
  return g.bias ? launch_kernel<AF, BF, true, false, kEpiPlain, BM, BN, WM, WN>(p, grid, device, stream)
                : launch_kernel<AF, BF, false, false, kEpiPlain, BM, BN, WM, WN>(p, grid, device, stream);
}

// Split-K launch: 256x256 tiles, grid = tiles * splits (one batch), bf16 output with an optional
// bias.  The workspace holds a counter and a ready flag per tile (zero on entry, left zero on
// exit) and then one fp32 partial tile per tile.
template <int AF, int BF>
hipError_t launch_split(const GemmProblem& g, const SplitPlan& plan, int device,
                         hipStream_t stream) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
  uint8_t* ws = static_cast<uint8_t*>(g.workspace);
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         (g.M + BM - 1) / BM, (g.N + BN - 1) / BN,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c,
         nullptr, nullptr, 0, 0, nullptr, 0,
         reinterpret_cast<float*>(ws + plan.counter_bytes), reinterpret_cast<uint32_t*>(ws),
         plan.splits};
  dim3 grid(p.tiles_m * p.tiles_n * plan.splits, 1);
  return g.bias ? launch_kernel<AF, BF, true, false, kEpiPlain, BM, BN, WM, WN, true>(p, grid, device, stream)
                : launch_kernel<AF, BF, false, false, kEpiPlain, BM, BN, WM, WN, true>(p, grid, device, stream);
}

template <int AF, int BF>
hipError_t launch_formats(const GemmProblem& g, const DeviceInfo& dev, hipStream_t stream) {
  if (g.workspace) {
    const SplitPlan plan = plan_split(g.M, g.N, g.K, g.batch);
    if (plan.splits > 1) {
      if (mx_kernel_takes(g.K, plan.splits)) return launch_gemm_mx(AF, BF, g, &plan, 256, stream);
      return launch_split<AF, BF>(g, plan, dev.device, stream);
    }
  }
  // Largest tile that still gives every CU a workgroup; the smallest one otherwise.
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  auto tiles = [&](int bm, int bn) {
    return static_cast<int64_t>((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn) * g.batch;
  };
  // Above half the CUs, one wave of 256x256 tiles beats the three or four waves of 128x128 tiles
  // the same output needs (a 128x128 step costs 0.37 of a 256x256 step for a quarter of the work).
  // Where 256x224 tiles fill the last wave better, the large kernel takes those (mx_tile_n).  On
  // 4096x7168 (448 tiles of 256x256: 1.75 waves of 256 CUs; 512 of 256x224: two full waves) that
  // raises the CUs' busy share of the kernel's cycles from 0.76 to 0.86 but the time stays within
  // 1%: with every CU busy the clock falls from 2.05 to 1.98 GHz (the chip is at its power limit
  // under this load), as it does for a partial last wave's idle CUs in reverse (its tiles run
  // faster per CU).
  if (2 * tiles(256, 256) > cus) {
    if (mx_kernel_takes(g.K, 1))
      return launch_gemm_mx(AF, BF, g, nullptr, mx_tile_n(g.M, g.N, g.batch, cus), stream);
    return launch_tile<AF, BF, 256, 256, 2, 4>(g, dev.device, stream);
  }
  if (tiles(128, 128) >= cus) return launch_tile<AF, BF, 128, 128, 2, 2>(g, dev.device, stream);
  // 64x64 tiles: with K of at most four chunks of 256 and one wave of workgroups, the kernel that
  // copies the tile's whole K into LDS at the start (gemm_small.hip) instead of staging it a step
  // at a time.  Its LDS (up to 128 KB) holds one workgroup per CU, so past one wave the step-wise
  // kernel, several of whose workgroups share a CU, is faster (measured).
  if (small_kernel_takes(g.K) && tiles(64, 64) <= cus) return launch_gemm_small(AF, BF, g, stream);
  return launch_tile<AF, BF, 64, 64, 2, 2>(g, dev.device, stream);
}

}  // namespace

hipError_t launch_gemm_bf16(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                            hipStream_t stream) {
  if (a_fmt == kFp8 && b_fmt == kFp4) return launch_formats<kFp8, kFp4>(p, dev, stream);
  if (a_fmt == kFp8 && b_fmt == kFp8) return launch_formats<kFp8, kFp8>(p, dev, stream);
  if (a_fmt == kFp4 && b_fmt == kFp4) return launch_formats<kFp4, kFp4>(p, dev, stream);
  if (a_fmt == kBf8 && b_fmt == kFp8Rows) return launch_formats<kBf8, kFp8Rows>(p, dev, stream);
  return hipErrorInvalidValue;
}

}  // namespace mx
