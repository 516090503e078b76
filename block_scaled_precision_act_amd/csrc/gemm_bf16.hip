// Block-scaled GEMM with FP8 operands for gfx950: decode to exact bf16, contract on the bf16
// MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation, fused fp32 bias, one bf16 rounding.
//
// What is computed ("formats.py" page: decode_fp4 / decode_fp8_block / act_qdq; "AstrAI commit
// log" page: bias added in fp32 before the single bf16 rounding):
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
// Design (per workgroup of 4 wavefronts, tile BM x BN, K step 64):
//   * global -> registers: 16-byte loads of the raw codes (FP8: 16 values, FP4: 32 values) and the
//     E8M0 byte of their 32-block, issued one K step ahead of the MFMAs that consume them;
//   * registers -> LDS: v_cvt_scalef32_pk_bf16_{fp8,fp4} decode two values per instruction with
//     the scale folded in; rows are 128 B (64 bf16) with the 16-byte chunk index XOR-swizzled by
//     the row (chunk c of row r lives at c ^ (r & 7)), so the 32 rows one MFMA operand read
//     touches hit 8 distinct chunk positions per 8 lanes: no bank conflicts;
//   * two LDS stages, one barrier per K step: the next stage is written while the current one is
//     read, and the barrier at the end of the step orders both;
//   * wavefront tile (BM/2) x (BN/2) of 32x32 MFMA blocks held in accumulator registers;
//   * the workgroup -> tile map keeps consecutive tiles on one XCD (workgroups are dealt to the 8
//     XCDs round-robin) and walks them in groups of GROUP_M tile rows, so an XCD's L2 holds the
//     A rows and B rows its running tiles share.
#include "mx_internal.h"

namespace mx {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

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

constexpr int kBK = 64;          // K elements per stage
constexpr int kRowBytes = 128;   // one LDS row: 64 bf16
constexpr int kGroupM = 8;

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
};

// fp32 value of an E8M0 byte (2^(b-127)); byte 0 is the fp32 subnormal 2^-127.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

__device__ __forceinline__ uint32_t pk_bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// 16 E4M3 codes times s -> 16 bf16 (two 16-byte chunks, element order preserved).
__device__ __forceinline__ void decode_fp8(uint4 v, float s, uint4& o0, uint4& o1) {
  o0.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, s, false));
  o0.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, s, true));
  o0.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, s, false));
  o0.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, s, true));
  o1.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.z, s, false));
  o1.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.z, s, true));
  o1.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.w, s, false));
  o1.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.w, s, true));
}

// 8 E2M1 codes (one dword, low nibble first) times s -> 8 bf16 (one 16-byte chunk).
__device__ __forceinline__ uint4 decode_fp4_dword(uint32_t d, float s) {
  uint4 o;
  o.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0));
  o.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1));
  o.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2));
  o.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3));
  return o;
}

// LDS rows are 128 B (64 bf16 = 8 chunks of 16 B).  Chunk c of row r is stored at chunk
// c ^ swz(r), swz(r) = (r & 7) ^ parity(bits 1..3 of r), period 16 in r.  It keeps every LDS pass
// free of bank conflicts for all three access patterns, whether a pass serves 8 lanes (128 B of
// banks) or 16 lanes (256 B): the fragment reads (8 or 16 consecutive rows at one logical chunk),
// the FP8 decode writes (rows r, r+1 x 4 pieces of 2 chunks) and the FP4 decode writes (rows
// r..r+3 x 2 pieces of 4 chunks).  Found by exhaustive search over period-16 tables.
__device__ __forceinline__ int swz(int row) {
  return (row & 7) ^ (__builtin_popcount((row >> 1) & 7) & 1);
}

__device__ __forceinline__ uint32_t lds_offset(int row, int chunk) {
  return static_cast<uint32_t>(row * kRowBytes + ((chunk ^ swz(row)) << 4));
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  bf16x2 p = {static_cast<__bf16>(v), static_cast<__bf16>(0.0f)};
  return static_cast<uint16_t>(pk_bits(p) & 0xFFFFu);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // Raw buffer (stride 0) with a byte bound: loads at or past `bytes` return zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Raw codes one thread carries from global memory to LDS for one operand.
// A row of one K step is FP8: 4 pieces of 16 codes; FP4: 2 pieces of 32 codes (16 bytes each).
// Thread t owns pieces c = t + i*NT (i < kPer): row c / kPieces, piece c % kPieces.  Rows past
// the matrix and the K half past the end of a partial last step read zeros through the buffer
// bound; the per-step advance is a scalar offset.  Each piece is decoded into LDS in one part of
// a K step and reloaded right after, for the step after next, so every piece has a whole K step
// to arrive with a single register set.
template <int FMT, int ROWS, int NT, int POFF>
struct Stager {
  static constexpr int kPieces = FMT == kFp8 ? 4 : 2;
  static constexpr int kStepBytes = FMT == kFp8 ? 64 : 32;       // bytes of a row per K step
  static constexpr int kTotal = ROWS * kPieces;
  static constexpr int kPer = (kTotal + NT - 1) / NT;
  static constexpr bool kAll = kTotal % NT == 0;
  static constexpr int kRowStride = NT / kPieces;                // rows between pieces i, i+1
  static constexpr int kChunksPerPiece = FMT == kFp8 ? 2 : 4;    // 16-byte bf16 chunks
  static constexpr int kChunks = kPer * kChunksPerPiece;
  static constexpr uint32_t kOob = 0x80000000u;                  // past any buffer bound
  static_assert(NT % kPieces == 0 && kRowStride % 16 == 0, "swizzle period");

  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t voff[kPer];      // byte offset of piece i at K step 0
  uint32_t soff[kPer];      // byte offset of its scale byte at K step 0
  uint32_t lds0;            // LDS offset (stage-relative) of piece 0's first chunk
  bool upper;               // the thread's pieces cover K [32, 64) of a step
  uint4 raw[kPer];
  uint32_t sbyte[kPer];

  __device__ __forceinline__ void init(const uint8_t* base, const uint8_t* sbase, int row0,
                                       int rows_valid, int K, bool block_scales, int lds_row0) {
    const int pitch = FMT == kFp8 ? K : K / 2;
    const int kb_total = K / 32;
    const int t = threadIdx.x;
    const int p = t % kPieces;
    const int koff = (FMT == kFp8 ? 16 : 32) * p;
    upper = koff >= 32;
    const int srows = block_scales ? (rows_valid + 31) / 32 : rows_valid;
    codes = make_rsrc(base, static_cast<uint32_t>(rows_valid) * static_cast<uint32_t>(pitch));
    scales = make_rsrc(sbase, static_cast<uint32_t>(srows) * static_cast<uint32_t>(kb_total));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = min(row0 + t / kPieces + i * kRowStride, rows_valid);   // == rows_valid: OOB
      voff[i] = static_cast<uint32_t>(r) * pitch + 16 * p;
      const int sr = block_scales ? r / 32 : r;
      soff[i] = static_cast<uint32_t>(sr) * kb_total + koff / 32;
    }
    lds0 = lds_offset(lds_row0 + t / kPieces, kChunksPerPiece * p);
  }

  // Loads piece I of K step kt; `partial` marks a last step holding only 32 valid K.
  template <int I>
  __device__ __forceinline__ void load_piece(int kt, bool partial) {
    const uint32_t v = (partial && upper) ? kOob : voff[I];
    raw[I] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(codes, v, kt * kStepBytes, 0));
    __builtin_amdgcn_sched_barrier(0);
    sbyte[I] = __builtin_amdgcn_raw_buffer_load_b8(scales, soff[I], kt * 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ void load_all(int kt, bool partial) {
    static_for<0, kPer>([&](auto ic) { load_piece<decltype(ic)::value>(kt, partial); });
  }

  // The quarter of a K step (sub-step) in which piece i is decoded, all its chunks at once; A and
  // B pieces are offset by POFF so they alternate.  A piece is reloaded at the end of its quarter
  // and decoded again in the same quarter of the next step: a whole step of latency.
  static constexpr int piece_part(int i) { return ((i * 4) / kPer + POFF) % 4; }
  static constexpr int part_of(int q) { return piece_part(q / kChunksPerPiece); }

  // Decodes chunk Q and writes it to the LDS stage.  The chunks of one piece are consecutive
  // logical chunks of one row: the physical chunk of logical (base + j) is (base ^ swz) ^ j
  // because base is a multiple of kChunksPerPiece.
  template <int Q>
  __device__ __forceinline__ void store_chunk(uint8_t* stage) const {
    constexpr int i = Q / kChunksPerPiece, j = Q % kChunksPerPiece;
    if (!kAll && !(static_cast<int>(threadIdx.x) + i * NT < kTotal)) return;
    const float s = e8m0_value(sbyte[i]);
    const uint32_t c0 = (lds0 >> 4) & 7;
    uint8_t* dst = stage + (lds0 - (c0 << 4)) + i * kRowStride * kRowBytes + ((c0 ^ j) << 4);
    uint4 o;
    if (FMT == kFp8) {
      const uint32_t lo = j == 0 ? raw[i].x : raw[i].z;
      const uint32_t hi = j == 0 ? raw[i].y : raw[i].w;
      o.x = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, false));
      o.y = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, true));
      o.z = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, false));
      o.w = pk_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, true));
    } else {
      const uint32_t d = j == 0 ? raw[i].x : j == 1 ? raw[i].y : j == 2 ? raw[i].z : raw[i].w;
      o = decode_fp4_dword(d, s);
    }
    *reinterpret_cast<uint4*>(dst) = o;
  }

  template <int PART>
  static constexpr int chunks_in_part() {
    int n = 0;
    for (int q = 0; q < kChunks; ++q) n += part_of(q) == PART ? 1 : 0;
    return n;
  }

  // Part PART of a step's decode + store.
  template <int PART>
  __device__ __forceinline__ void store_part(uint8_t* stage) const {
    static_for<0, kChunks>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      if constexpr (part_of(q) == PART) store_chunk<q>(stage);
    });
  }

  // The reloads after part PART: every piece whose last chunk was decoded in that part, in a
  // fixed order (each load is fenced from the scheduler), so every path into the K loop,
  // prologue included, leaves the same sequence of outstanding loads and the waits the loop
  // needs stay as shallow as the data dependences allow.
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

// Tile coordinates of workgroup `bid` out of `nb`: XCD-contiguous, then grouped by GROUP_M rows.
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

template <int TM, int TN>
struct Frags {
  bf16x8 a[2][TM], b[2][TN];
};

template <int TM, int TN, int BUF>
__device__ __forceinline__ void read_frags(const uint8_t* stage, uint32_t a_base, uint32_t b_base,
                                           uint32_t coff, Frags<TM, TN>& f) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
    f.a[BUF][i] = *reinterpret_cast<const bf16x8*>(stage + a_base + i * 32 * kRowBytes + coff);
#pragma unroll
  for (int j = 0; j < TN; ++j)
    f.b[BUF][j] = *reinterpret_cast<const bf16x8*>(stage + b_base + j * 32 * kRowBytes + coff);
}

// One K step on LDS stage `cur`: four 16-wide sub-steps.  FRAG_DB: each sub-step reads the next
// sub-step's fragments ahead of its own MFMAs.  When STORE, sub-step ks also decodes part ks of
// the next step's codes into `nxt` and, at its end (LOAD), reloads the finished pieces for step
// kt_load.
// Scheduling groups ask for every MFMA to be followed by a slice of the sub-step's other work, so
// the matrix pipe keeps issuing while the VALU decodes and the LDS reads and writes proceed; a
// scheduling fence closes each sub-step so later fragments are not hoisted (and kept live) early.
template <bool STORE, bool LOAD, bool FRAG_DB, int TM, int TN, class SA, class SB>
__device__ __forceinline__ void k_step(const uint8_t* cur, uint8_t* nxt, uint32_t a_base,
                                       uint32_t b_base, const uint32_t (&coff)[4], SA& sa, SB& sb,
                                       v16f (&acc)[TM][TN], int kt_load, bool partial_load) {
  Frags<TM, TN> f;
  if constexpr (FRAG_DB) read_frags<TM, TN, 0>(cur, a_base, b_base, coff[0], f);
  static_for<0, 4>([&](auto ksc) {
    constexpr int ks = decltype(ksc)::value;
    constexpr int buf = FRAG_DB ? (ks & 1) : 0;
    if constexpr (FRAG_DB) {
      if constexpr (ks < 3) read_frags<TM, TN, (ks + 1) & 1>(cur, a_base, b_base, coff[ks + 1], f);
    } else {
      read_frags<TM, TN, 0>(cur, a_base, b_base, coff[ks], f);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[buf][i], f.b[buf][j],
                                                            acc[i][j], 0, 0, 0);
    if constexpr (STORE) {
      sa.template store_part<ks>(nxt);
      sb.template store_part<ks>(nxt);
    }
    // Interleave: each MFMA is followed by a slice of the sub-step's other instructions.
    constexpr int kM = TM * TN;
    constexpr int kReads = FRAG_DB ? (ks < 3 ? TM + TN : 0) : 0;
    constexpr int kChunksHere = STORE ? SA::template chunks_in_part<ks>() + SB::template chunks_in_part<ks>() : 0;
    constexpr int kCvt = 4 * kChunksHere;
    static_for<0, kM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
      constexpr int r0 = m * kReads / kM, r1 = (m + 1) * kReads / kM;
      if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);   // DS read
      constexpr int v0 = m * kCvt / kM, v1 = (m + 1) * kCvt / kM;
      if constexpr (v1 > v0) __builtin_amdgcn_sched_group_barrier(0x002, v1 - v0, 0);   // VALU
      constexpr int w0 = m * kChunksHere / kM, w1 = (m + 1) * kChunksHere / kM;
      if constexpr (w1 > w0) __builtin_amdgcn_sched_group_barrier(0x200, w1 - w0, 0);   // DS write
    });
    // Close the scheduling region: later sub-steps' reads must not be hoisted into this one.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (STORE && LOAD) {
      sa.template load_part<ks>(kt_load, partial_load);
      sb.template load_part<ks>(kt_load, partial_load);
    }
  });
}

template <int AF, int BF, bool BIAS, int BM, int BN, int WM, int WN, bool FRAG_DB>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(Args p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;     // WM x WN wavefronts
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static_assert(BM * BN * 2 <= 2 * kStageBytes, "the bf16 output tile must fit the operand stages");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wm = wave / WN, wn = wave % WN;

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t bz = blockIdx.y;
  const int m0 = tm * BM, n0 = tn * BN;

  Stager<AF, BM, NT, 0> sa;
  Stager<BF, BN, NT, 1> sb;
  sa.init(p.a + bz * p.stride_a, p.a_s + bz * p.stride_as, m0, p.M, p.K, false, 0);
  sb.init(p.b + bz * p.stride_b, p.b_s + bz * p.stride_bs, n0, p.N, p.K, BF == kFp8, BM);

  // Operand fragment offsets: rows wm*WTM + 32i + l32 (A) and BM + wn*WTN + 32j + l32 (B) share
  // swz(l32), so four chunk offsets (one per 16-wide K sub-step) serve every fragment.
  const uint32_t a_base = static_cast<uint32_t>((wm * WTM + l32) * kRowBytes);
  const uint32_t b_base = static_cast<uint32_t>((BM + wn * WTN + l32) * kRowBytes);
  uint32_t coff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) coff[ks] = static_cast<uint32_t>(((2 * ks + h) ^ swz(l32)) << 4);

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

  // Pipeline: step k's codes are decoded into LDS stage k & 1 during step k-1's MFMAs, piece by
  // piece, and each piece is reloaded for step k+1 right after its decode.
  const int KT = (p.K + kBK - 1) / kBK;
  const int last_partial = (p.K % kBK) != 0 ? KT - 1 : -1;
  sa.load_all(0, last_partial == 0);
  sb.load_all(0, last_partial == 0);
  sa.store_all(lds);
  sb.store_all(lds);
  if (KT > 1) {
    static_for<0, 4>([&](auto pc) {
      constexpr int P = decltype(pc)::value;
      sa.template load_part<P>(1, last_partial == 1);
      sb.template load_part<P>(1, last_partial == 1);
    });
  }
  __syncthreads();
  int kt = 0;
  for (; kt + 2 < KT; ++kt) {
    k_step<true, true, FRAG_DB>(lds + (kt & 1) * kStageBytes, lds + ((kt + 1) & 1) * kStageBytes,
                                a_base, b_base, coff, sa, sb, acc, kt + 2, kt + 2 == last_partial);
    __syncthreads();
  }
  if (kt + 1 < KT) {
    k_step<true, false, FRAG_DB>(lds + (kt & 1) * kStageBytes, lds + ((kt + 1) & 1) * kStageBytes,
                                 a_base, b_base, coff, sa, sb, acc, 0, false);
    __syncthreads();
    ++kt;
  }
  k_step<false, false, FRAG_DB>(lds + (kt & 1) * kStageBytes, lds, a_base, b_base, coff, sa, sb,
                                acc, 0, false);

  // Epilogue, staged through LDS: fp32 + bias, one bf16 rounding, written into a row-major bf16
  // tile [BM][BN] (16-byte chunk c of row r at chunk c ^ (4 * bit 2 of r): the two row groups a
  // wavefront writes in one pass, 4 rows apart, land in different halves of the bank space), then
  // copied out in coalesced 16-byte row segments.
  __syncthreads();                       // every wavefront is done reading the operand stages
  constexpr int kTileRow = BN * 2;       // bytes of one bf16 tile row
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int tcol = wn * WTN + 32 * j + l32;
    float bias = 0.0f;
    if (BIAS) {
      const int col = min(n0 + tcol, p.N - 1);
      bias = __uint_as_float(static_cast<uint32_t>(p.bias[bz * p.stride_bias + col]) << 16);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int trow = wm * WTM + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);   // rows trow, trow+1
        bf16x2 pk = {static_cast<__bf16>(acc[i][j][r] + bias), static_cast<__bf16>(acc[i][j][r + 1] + bias)};
        const uint32_t w = pk_bits(pk);
        const int ch = (tcol >> 3) ^ (((trow >> 2) & 1) << 2);
        const uint32_t off = static_cast<uint32_t>(trow * kTileRow + ch * 16 + (tcol & 7) * 2);
        *reinterpret_cast<uint16_t*>(lds + off) = static_cast<uint16_t>(w & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(lds + off + kTileRow) = static_cast<uint16_t>(w >> 16);
      }
    }
  }
  __syncthreads();
  constexpr int kChunksPerRow = BN / 8;
  uint16_t* c = p.c + bz * p.stride_c;
  for (int idx = threadIdx.x; idx < BM * kChunksPerRow; idx += NT) {
    const int trow = idx / kChunksPerRow, tch = idx % kChunksPerRow;
    const int row = m0 + trow, col = n0 + tch * 8;
    if (row >= p.M || col >= p.N) continue;
    const int ch = tch ^ (((trow >> 2) & 1) << 2);
    const uint4 v = *reinterpret_cast<const uint4*>(lds + trow * kTileRow + ch * 16);
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

template <int AF, int BF, int BM, int BN, int WM, int WN, bool FRAG_DB>
hipError_t launch_tile(const GemmProblem& g, hipStream_t stream) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         (g.M + BM - 1) / BM, (g.N + BN - 1) / BN,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c};
  constexpr int kLds = 2 * (BM + BN) * kRowBytes;
  dim3 grid(p.tiles_m * p.tiles_n, g.batch);
  auto k = g.bias ? gemm_bf16_kernel<AF, BF, true, BM, BN, WM, WN, FRAG_DB>
                  : gemm_bf16_kernel<AF, BF, false, BM, BN, WM, WN, FRAG_DB>;
  // The dynamic-LDS limit is raised once per kernel (above 64 KB needs the attribute).
  static const hipError_t attr_ok = [] {
    hipError_t e1 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gemm_bf16_kernel<AF, BF, true, BM, BN, WM, WN, FRAG_DB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    hipError_t e2 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gemm_bf16_kernel<AF, BF, false, BM, BN, WM, WN, FRAG_DB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    return e1 != hipSuccess ? e1 : e2;
  }();
  if (attr_ok != hipSuccess) return attr_ok;
  hipLaunchKernelGGL(k, grid, dim3(64 * WM * WN), kLds, stream, p);
  return hipGetLastError();
}

template <int AF, int BF>
hipError_t launch_formats(const GemmProblem& g, const DeviceInfo& dev, hipStream_t stream) {
  // Largest tile that still gives every CU a workgroup; the smallest one otherwise.
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  auto tiles = [&](int bm, int bn) {
    return static_cast<int64_t>((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn) * g.batch;
  };
  // A last partial wave of 256x256 tiles is not worth splitting further: on 4096x7168 (448 tiles,
  // 1.75 waves) the 192 tiles of the second wave run 18% faster per CU than a full wave does, and
  // finishing them as 256 tiles of 256x192 in a second launch measured the same total time.
  if (tiles(256, 256) >= cus) return launch_tile<AF, BF, 256, 256, 4, 2, true>(g, stream);
  if (tiles(128, 128) >= cus) return launch_tile<AF, BF, 128, 128, 2, 2, true>(g, stream);
  return launch_tile<AF, BF, 64, 64, 2, 2, false>(g, stream);
}

}  // namespace

hipError_t launch_gemm_bf16(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                            hipStream_t stream) {
  if (a_fmt == kFp8 && b_fmt == kFp4) return launch_formats<kFp8, kFp4>(p, dev, stream);
  if (a_fmt == kFp8 && b_fmt == kFp8) return launch_formats<kFp8, kFp8>(p, dev, stream);
  if (a_fmt == kFp4 && b_fmt == kFp4) return launch_formats<kFp4, kFp4>(p, dev, stream);
  return hipErrorInvalidValue;
}

}  // namespace mx
