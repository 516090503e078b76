// Block-scaled GEMM with FP8 operands for gfx950, large problems: 256x256 output tiles, one
// wavefront per SIMD, operands staged raw into LDS by direct-to-LDS loads and decoded to exact
// bf16 in registers by every wavefront that contracts them.
//
// What is computed is the same as in gemm_bf16.hip ("formats.py" page: decode_fp4 /
// decode_fp8_block / act_qdq give the decoded operands; "AstrAI commit log" page: the bias joins
// the fp32 sum, which is rounded to bf16 once):
//   C[m,n] = bf16_rne( sum_k A[m,k] B[n,k] + bias[n] ),
// with A and B decoded exactly to bf16 (a 4-bit E4M3 or 2-bit E2M1 significand times the E8M0
// power of two is a bf16 value) and contracted on the bf16 MFMA (v_mfma_f32_32x32x16_bf16),
// which forms exact products and accumulates in fp32.
//
// Why this layout (measured on gfx950): an LDS write instruction costs the CU far more than a
// read of the same bytes, and a tile kernel that decodes A into LDS as bf16 and has eight
// wavefronts re-read it moves ~184 KB of LDS traffic per 64-wide K step of a 256x256 tile.  Here
// no wavefront writes LDS in the main loop:
//   * every K step, each operand's raw codes for the tile's 256 rows (E4M3/E5M2: 64 bytes a row,
//     E2M1: 32) are copied global -> LDS by buffer loads with the LDS as destination, into one of
//     four stages (separate LDS arrays, so the compiler's wait counting can tell a copy into one
//     stage from a read of another);
//   * the 4 wavefronts form a 2 x 2 grid; each owns a 128 x 128 tile (4 x 4 blocks of 32 x 32,
//     256 fp32 accumulators a lane) and reads the raw codes of its own 128 A rows and 128 B rows
//     (48-64 KB for the workgroup per step) and decodes each sub-step's 8 values per row with
//     v_cvt_scalef32_pk_bf16_{fp8,bf8,fp4}, the E8M0 scale folded in.  Decoding is repeated in
//     the two wavefronts that share a row: 128 converts per wavefront and step, which one
//     wavefront's 64 MFMAs of 32 cycles hide (measured);
//   * K order inside a step: lane group h of sub-step s contracts K [32h + 8s, 32h + 8s + 8) of
//     the step, for A and for B (a permutation of K, so the sum is unchanged), so a lane decodes
//     one whole 32-block of its row per step with one scale byte;
//   * the step's copy for step k + 3 is issued after the step's one barrier, so a copy has two
//     steps to land; scale bytes are loaded per lane into registers with the same lead;
//   * one barrier per step, in the middle: before it every wavefront waits for its copies of
//     the next step (vmcnt, counted exactly: each step issues the same number of loads); after
//     it the first reads of the next stage and the copies into the stage freed one step ago;
//   * the work of a sub-step (raw reads, decodes, copies, scale loads) is spread over the slots
//     between its 16 MFMAs, each slot fenced from the scheduler, so the matrix pipe gets an MFMA
//     between every few other instructions.
// The tile map, split-K handoff and epilogue are the ones gemm_bf16.hip uses (gemm_common.h);
// the epilogue stages the bf16 tile through the four (then idle) operand stages.
#include "gemm_common.h"

namespace mx {
namespace {

constexpr int kTile = 256;                 // BM = BN
constexpr int kWaves = 4;                  // 2 x 2
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;
constexpr int kStageBytes = 32768;         // A region (256 rows x 64 B), then B region
constexpr int kBRegion = 16384;
constexpr uint32_t kOob = 0x80000000u;     // past any buffer bound

// Wavefront grid and 32 x 32 blocks per wavefront of a 256 x BN output tile: 256 x 256 as 2 x 2
// wavefronts of 128 x 128 (4 x 4 blocks); 256 x 224 as 4 x 1 wavefronts of 64 x 224 (2 x 7
// blocks), for problems whose 256-wide tiles leave the last wave of workgroups part-empty.
template <int BN>
struct Shape {
  static_assert(BN == 256 || BN == 224, "tile width");
  static constexpr int kWM = BN == 256 ? 2 : 4;
  static constexpr int kWN = kWaves / kWM;
  static constexpr int kTM = kTile / kWM / 32;
  static constexpr int kTN = BN / kWN / 32;
};

// Bytes of one operand row per K step (64 K).
template <int FMT>
constexpr int step_bytes() { return byte_codes(FMT) ? 64 : 32; }

// Raw rows are stored with their 16-byte units swizzled: unit u of row r at u ^ unit_swz(r).
// Rows of 64 B: 16 consecutive rows reading one logical unit hit 16 distinct 16-byte bank
// groups; rows of 32 B likewise with the swizzle on row bit 3.  Period 16 (or 16) in r, and only
// row bits 2..3 matter, so row offsets that are multiples of 32 keep a lane's swizzle.
template <int FMT>
__device__ __forceinline__ int unit_swz(int r) {
  return byte_codes(FMT) ? (r >> 2) & 3 : (r >> 3) & 1;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS copy of one operand's raw codes, 256 rows per K step.  Wavefront w, copy j
// writes the 1 KB at stage offset (w * kPer + j) * 1024; its lane i fetches the 16 bytes that
// belong at byte 16 i of that KB (row and physical unit from the offset, logical unit through
// the swizzle).  The step's byte offset goes in the scalar offset, so a copy costs no vector
// instruction; rows past the matrix or past the tile's `rows_tile` read zeros through the buffer
// bound (their vector offset is past it), and so does every lane of a step past the range (bit
// 31 set by `oob`).
template <int FMT>
struct Copier {
  static constexpr int kRB = step_bytes<FMT>();
  static constexpr int kPer = kTile * kRB / 1024 / kWaves;    // copies per wavefront and step
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[kPer];       // row * pitch + 16 u, or kOob
  uint32_t lds_off[kPer];    // stage-relative LDS byte offset of copy j (wavefront-uniform)

  __device__ __forceinline__ void init(const uint8_t* base, int row0, int rows_valid, int rows_tile,
                                       int K, int wave, int lane, uint32_t region) {
    const uint32_t pitch = byte_codes(FMT) ? K : K / 2;
    rsrc = make_rsrc(base, static_cast<uint32_t>(rows_valid) * pitch);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int chunk = wave * kPer + j;
      const int byte = chunk * 1024 + 16 * lane;
      const int r = byte / kRB;
      const int u = ((byte % kRB) >> 4) ^ unit_swz<FMT>(r);
      const int row = row0 + r;
      voff[j] = r < rows_tile && row < rows_valid ? static_cast<uint32_t>(row) * pitch + 16u * u : kOob;
      lds_off[j] = region + static_cast<uint32_t>(chunk) * 1024u;
    }
  }

  template <int J>
  __device__ __forceinline__ void issue(uint8_t* stage, int kabs, uint32_t oob) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(stage + lds_off[J]), 16,
                                             static_cast<int>(voff[J] | oob), kabs * kRB, 0, 0);
  }
};

// kOob for a step at or past the end of the range (every lane of its loads reads zeros).
__device__ __forceinline__ uint32_t past(int kabs, int k_end) { return kabs >= k_end ? kOob : 0u; }

// Keeps a decoded operand where it is computed: the empty asm uses and redefines the value, so
// no pass can sink its converts past the scheduling fences to the MFMA that reads it.
__device__ __forceinline__ void pin(bf16x8& v) {
  v4u u = __builtin_bit_cast(v4u, v);
  asm volatile("" : "+v"(u));
  v = __builtin_bit_cast(bf16x8, u);
}

// One wavefront's view of one operand: NB blocks of 32 rows (rows row_w + 32 i + l32).  Per K
// step the lane reads the raw codes of the 32-block h of its row: E4M3/E5M2 two 16-byte units
// (u = 2h: sub-steps 0-1, kept in raw[0]; u = 2h + 1: sub-steps 2-3, raw[1]), E2M1 one (u = h,
// all four sub-steps, in raw[step parity]).  Scale bytes come a group of 4 steps at a time: one
// 8-byte load per block holds the group's 8 bytes of the lane's row (steps k..k+3, blocks h = 0
// and 1 each), kept in one of two register sets by group parity.
template <int FMT, bool BLOCK_SCALES, int NB>
struct Frag {
  static constexpr int kRB = step_bytes<FMT>();
  static constexpr int kUnits = byte_codes(FMT) ? 2 : 1;
  uint32_t rd[kUnits];       // stage-relative LDS offset of block 0's unit q
  uint4 raw[2][NB];          // byte codes: unit 0 in raw[0]; E2M1: the unit, by step parity
  uint4 raw1[2][NB];         // byte codes: unit 1, by step parity
  __amdgpu_buffer_rsrc_t srsrc;
  uint32_t soff[NB];         // byte offset of block i's scale row (or kOob)
  uint2 sv[2][NB];           // scale bytes of a group: parity, block
  uint32_t hsh;              // 8 h: the lane's byte within a step's pair
  float sc[NB];              // scale values of the step being decoded

  __device__ __forceinline__ void init(const uint8_t* sbase, int row0, int rows_valid, int kb,
                                       int row_w, int l32, int h, uint32_t region) {
    const int r = row_w + l32;
#pragma unroll
    for (int q = 0; q < kUnits; ++q) {
      const int u = byte_codes(FMT) ? 2 * h + q : h;
      rd[q] = region + static_cast<uint32_t>(r * kRB + ((u ^ unit_swz<FMT>(r)) << 4));
    }
    const int srows = BLOCK_SCALES ? (rows_valid + 31) / 32 : rows_valid;
    srsrc = make_rsrc(sbase, static_cast<uint32_t>(srows) * static_cast<uint32_t>(kb));
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int row = row0 + row_w + 32 * i + l32;
      const int sr = BLOCK_SCALES ? row / 32 : row;
      soff[i] = sr < srows ? static_cast<uint32_t>(sr) * kb : kOob;
    }
    hsh = 8u * h;
  }

  // Unit Q (byte codes) of block I of a step with parity PAR, from `stage`.
  template <int Q, int I, int PAR>
  __device__ __forceinline__ void read(const uint8_t* stage) {
    const uint4 v = *reinterpret_cast<const uint4*>(stage + rd[byte_codes(FMT) ? Q : 0] + I * 32 * kRB);
    if constexpr (!byte_codes(FMT)) raw[PAR][I] = v;
    else if constexpr (Q == 0) raw[0][I] = v;
    else raw1[PAR][I] = v;
  }

  // The scale bytes of block I for the group of steps starting at absolute step kabs0.
  template <int GP, int I>
  __device__ __forceinline__ void load_group(int kabs0, uint32_t oob) {
    sv[GP][I] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                              srsrc, soff[I] | oob, 2 * kabs0, 0));
  }

  // Scale values of step SP of the group held in set GP.
  template <int GP, int SP>
  __device__ __forceinline__ void take_scales() {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t d = SP < 2 ? sv[GP][i].x : sv[GP][i].y;
      sc[i] = e8m0_value((d >> (16u * (SP & 1) + hsh)) & 0xFFu);
    }
  }

  // bf16 operand of block I for sub-step S of a step with parity PAR.
  template <int S, int I, int PAR>
  __device__ __forceinline__ bf16x8 decode() const {
    uint4 o;
    if constexpr (FMT == kFp4) {
      const uint4 q = raw[PAR][I];
      const uint32_t d = S == 0 ? q.x : S == 1 ? q.y : S == 2 ? q.z : q.w;
      o = decode_fp4_dword(d, sc[I]);
    } else {
      const uint4 q = S < 2 ? raw[0][I] : raw1[PAR][I];
      const uint32_t lo = (S & 1) ? q.z : q.x, hi = (S & 1) ? q.w : q.y;
      o = FMT == kBf8 ? decode_bf8_pair(lo, hi, sc[I]) : decode_fp8_pair(lo, hi, sc[I]);
    }
    return __builtin_bit_cast(bf16x8, o);
  }
};

template <int AF, int BF, int BN>
struct Pipe {
  static constexpr int TM = Shape<BN>::kTM, TN = Shape<BN>::kTN;
  static constexpr bool kBBlock = BF == kFp8;        // 32x32 block scales
  static constexpr int kCpA = Copier<AF>::kPer, kCpB = Copier<BF>::kPer;
  static constexpr int kCp = kCpA + kCpB;            // copies per wavefront and step
  // the step's copy list in four parts: parts 0-2 leave in sub-steps 1-3 of the step three
  // steps earlier, part 3 in sub-step 0 of the step two steps earlier
  static constexpr int cut(int q) { return q * kCp / 4; }
  Copier<AF> ca;
  Copier<BF> cb;
  Frag<AF, false, TM> fa;
  Frag<BF, kBBlock, TN> fb;
  bf16x8 opa[2][TM], opb[2][TN];   // decoded operands, by sub-step parity

  template <int C>
  __device__ __forceinline__ void copy(uint8_t* stage, int kabs, uint32_t oob) {
    if constexpr (C < kCpA) ca.template issue<C>(stage, kabs, oob);
    else cb.template issue<C - kCpA>(stage, kabs, oob);
  }
};

// Residual epilogue: the bf16 residual tile, copied global -> LDS during the last K steps into the
// operand stages as they fall free, already in the epilogue's tile layout (rows 64 s .. 64 s + 63
// in stage s, tile_chunk swizzle), so the epilogue reads it from LDS without a memory round trip
// of its own.  Each 64-row slice is kPer 1 KB copies per wavefront; lane i of copy j brings the
// 16-byte chunk stored at byte 16 i of the slice's KB number (wave * kPer + j).  The copies take
// the slots of the operand copies that steps past the range would issue (one load each, so every
// wait count of the loop is unchanged; a slot beyond kPer loads zeros into the stage's spare
// bytes), and the rest leave after the last step's barrier.  Only a tile inside the matrix with
// 16-byte aligned rows (`on`) reads its residual this way; for any other tile the buffer holds no
// bytes, so the same copies load zeros (no branch: the compiler's wait counting keeps telling
// the stages apart) and the epilogue loads the residual itself.
template <int BN>
struct ResTail {
  static constexpr int kChunks = BN / 8;                 // 16-byte chunks a tile row
  static constexpr int kSliceBytes = 64 * BN * 2;
  static constexpr int kPer = kSliceBytes / 1024 / kWaves;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t slice_bytes;      // 64 rows of the residual
  uint32_t pitch;            // N, in elements
  int wave, lane;
  bool on;

  __device__ __forceinline__ void init(const Args& p, int m0, int n0, int64_t bz, int wave_,
                                       int lane_) {
    const uint16_t* res = p.res + bz * p.stride_res;
    wave = wave_;
    lane = lane_;
    on = m0 + kTile <= p.M && n0 + BN <= p.N && (p.N & 7) == 0 &&
         (reinterpret_cast<uintptr_t>(res) & 15u) == 0 && p.N <= (1 << 22);
    pitch = static_cast<uint32_t>(p.N);
    slice_bytes = 128u * pitch;
    rsrc = make_rsrc(on ? res + static_cast<int64_t>(m0) * p.N + n0 : res,
                     on ? (255u * pitch + BN) * 2u : 0u);
  }

  // Copy J of slice `slice` into `stage`; J >= kPer: zeros into the stage's spare bytes.
  template <int J, int kCp>
  __device__ __forceinline__ void issue(uint8_t* stage, int slice) const {
    if constexpr (J < kPer) {
      const int q = (wave * kPer + J) * 64 + lane;          // stored chunk within the slice
      const int r = q / kChunks;
      const int c = tile_chunk<kChunks>(r, q % kChunks);    // the chunk it holds
      const uint32_t voff = (static_cast<uint32_t>(r) * pitch + 8u * c) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_ptr_t)(stage + (wave * kPer + J) * 1024), 16, static_cast<int>(voff),
          static_cast<int>(slice * slice_bytes), 0, 0);
    } else {
      constexpr int kFill = kCp - kPer;
      static_assert(kSliceBytes + kWaves * kFill * 1024 <= kStageBytes, "stage spare bytes");
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_ptr_t)(stage + kSliceBytes + (wave * kFill + (J - kPer)) * 1024), 16,
          static_cast<int>(kOob), 0, 0, 0);
    }
  }
};

// s_waitcnt operand: vmcnt(n) lgkmcnt(0), expcnt at its maximum (gfx9 encoding).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// One K step.  P8 = the step's index modulo 8 (the loop runs 8 steps per iteration, so that
// every stage, register set and wait count is named at compile time): stage P8 % 4, scale group
// P8 / 4 of the iteration (register set parity), step P8 % 4 within it.  kl is the step's index
// within the range, k0 the range's first absolute step, k_end its end.
// The step's barrier follows sub-step 0.  Before it every wavefront waits until the copies of
// the next step have landed; after it the next step's raw codes are read (unit 0 in sub-step 1,
// unit 1 in sub-step 2), a sub-step or two before they are decoded.
// Loads (vector memory), spread over the window between two barriers: in sub-steps 1-3 parts
// 0-2 of the copies of step kl + 3, in sub-step 0 part 3 of the copies of step kl + 2; when kl
// is the first step of a scale group, the next group's scale bytes in sub-step 2.
// Tasks within a sub-step, in order, spread over the slots after its TM x TN MFMAs: raw reads,
// the next step's scale values (sub-step 3), decodes of the next sub-step (sub-step 3: the next
// step's sub-step 0), copies, scale loads.
// TAIL: the range's last 8 steps in a kernel with the residual epilogue.  The copy slots of
// steps past the range bring the residual tile (ResTail); the scale group past the range is not
// loaded (its registers would be dead, and the compiler, reusing them, would wait for the loads);
// the last step reads and decodes nothing for the step after it, and after its barrier the
// residual copies with no slot leave: those of slice 2 that would have gone in the next step's
// sub-step 0, those beyond a slice's slots, and slice 3, whose stage falls free at that barrier.
template <int P8, bool TAIL, int AF, int BF, int BN>
__device__ __forceinline__ void mx_step(Pipe<AF, BF, BN>& P, const ResTail<BN>& R,
                                        uint8_t* const (&st)[kStages],
                                        v16f (&acc)[Shape<BN>::kTM][Shape<BN>::kTN], int k0,
                                        int kl, int k_end) {
  using PP = Pipe<AF, BF, BN>;
  using RT = ResTail<BN>;
  constexpr bool kLast = TAIL && P8 == 7;
  constexpr int kM = PP::kCp < RT::kPer ? PP::kCp : RT::kPer;   // slots that carry residual
  constexpr int kC3 = PP::cut(3);
  constexpr int kLeft = RT::kPer - kM;                           // per slice, beyond the slots
  constexpr int kPart3 = kM > kC3 ? kM - kC3 : 0;                // slice 2's sub-step-0 part
  constexpr int kExtra = kLast ? 3 * kLeft + kPart3 + RT::kPer : 0;
  constexpr int TM = PP::TM, TN = PP::TN, NM = TM * TN;
  constexpr int ST = P8 % kStages;
  constexpr int ST1 = (ST + 1) % kStages;
  constexpr int PAR = ST & 1, PAR1 = ST1 & 1;
  constexpr int SP = P8 % 4, GP = P8 / 4;            // step within its scale group, group parity
  constexpr int N8 = (P8 + 1) % 8;                   // the next step's position
  constexpr bool kByteA = byte_codes(AF), kByteB = byte_codes(BF);
  const uint8_t* nxt = st[ST1];
  const int kabs = k0 + kl;
  const uint32_t oob2 = past(kabs + 2, k_end), oob3 = past(kabs + 3, k_end);
  const uint32_t oobg = past(kabs + 4, k_end);
  static_for<0, 4>([&](auto sc_) {
    constexpr int s = decltype(sc_)::value;
    constexpr int nb = (s + 1) & 1;          // operand buffer filled during sub-step s
    constexpr int ds = (s + 1) & 3;          // sub-step decoded (s == 3: the next step's 0)
    constexpr int dpar = s == 3 ? PAR1 : PAR;
    // raw reads of the next step: unit 0 (and the one E2M1 unit) in s = 1, unit 1 in s = 2
    constexpr int kRdA = !kLast && (s == 1 || (s == 2 && kByteA)) ? TM : 0;
    constexpr int kRdB = !kLast && (s == 1 || (s == 2 && kByteB)) ? TN : 0;
    constexpr int kScl = s == 3 && !kLast ? 1 : 0;
    constexpr int kDec = s == 3 && kLast ? 0 : TM + TN;
    constexpr int c0 = s == 0 ? PP::cut(3) : PP::cut(s - 1);
    constexpr int c1 = s == 0 ? PP::kCp : PP::cut(s);
    constexpr int kCpy = c1 - c0;
    constexpr int e0 = s == 0 ? 0 : (s - 1) * kExtra / 3, e1 = s == 0 ? 0 : s * kExtra / 3;
    constexpr int kExt = e1 - e0;
    // (TAIL: no scale bytes for the group past the range, whose step 4 would load them)
    constexpr int kSld = (s == 2 && SP == 0 && !(TAIL && P8 == 4)) ? TM + TN : 0;
    constexpr int kTasks = kRdA + kRdB + kScl + kDec + kCpy + kExt + kSld;
    auto task = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if constexpr (t < kRdA) {
        P.fa.template read<s == 1 ? 0 : 1, t, PAR1>(nxt);
      } else if constexpr (t < kRdA + kRdB) {
        P.fb.template read<s == 1 ? 0 : 1, t - kRdA, PAR1>(nxt);
      } else if constexpr (t < kRdA + kRdB + kScl) {
        P.fa.template take_scales<N8 / 4, N8 % 4>();
        P.fb.template take_scales<N8 / 4, N8 % 4>();
      } else if constexpr (t < kRdA + kRdB + kScl + kDec) {
        constexpr int d = t - kRdA - kRdB - kScl;
        if constexpr (d < TM) {
          P.opa[nb][d] = P.fa.template decode<ds, d, dpar>();
          pin(P.opa[nb][d]);
        } else {
          P.opb[nb][d - TM] = P.fb.template decode<ds, d - TM, dpar>();
          pin(P.opb[nb][d - TM]);
        }
      } else if constexpr (t < kRdA + kRdB + kScl + kDec + kCpy) {
        constexpr int c = c0 + t - (kRdA + kRdB + kScl + kDec);
        if constexpr (s >= 1) {
          if constexpr (TAIL && P8 >= 5) R.template issue<c, PP::kCp>(st[(ST + 3) % kStages], P8 - 5);
          else P.template copy<c>(st[(ST + 3) % kStages], kabs + 3, oob3);
        } else {
          if constexpr (TAIL && P8 >= 6) R.template issue<c, PP::kCp>(st[(ST + 2) % kStages], P8 - 6);
          else P.template copy<c>(st[(ST + 2) % kStages], kabs + 2, oob2);
        }
      } else if constexpr (t < kRdA + kRdB + kScl + kDec + kCpy + kExt) {
        // residual copies without a slot (kLast): slices 0-2 beyond their slots, slice 2's
        // sub-step-0 part, then slice 3
        constexpr int e = e0 + t - (kRdA + kRdB + kScl + kDec + kCpy);
        constexpr int sl = e < 3 * kLeft ? e / kLeft : e < 3 * kLeft + kPart3 ? 2 : 3;
        constexpr int c = e < 3 * kLeft ? kM + e % kLeft
                          : e < 3 * kLeft + kPart3 ? kC3 + (e - 3 * kLeft)
                                                   : e - 3 * kLeft - kPart3;
        R.template issue<c, PP::kCp>(st[sl], sl);
      } else {
        constexpr int q = t - (kRdA + kRdB + kScl + kDec + kCpy + kExt);
        if constexpr (q < TM) P.fa.template load_group<GP ^ 1, q>(kabs + 4, oobg);
        else P.fb.template load_group<GP ^ 1, q - TM>(kabs + 4, oobg);
      }
    };
    static_for<0, NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int i = m / TN, j = m % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(P.opb[s & 1][j], P.opa[s & 1][i],
                                                          acc[i][j], 0, 0, 0);
      static_for<m * kTasks / NM, (m + 1) * kTasks / NM>(task);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (s == 0) {
      // Every wavefront's copies of the next step have landed: still in flight may be only the
      // loads of the window since the previous barrier, i.e. the copies of step kl + 2 and the
      // scale group the previous step issued, if it did.  And every read of the stages the
      // copies of this window overwrite is done.
      constexpr int kAfter = PP::kCp + ((P8 + 7) % 4 == 0 && !(TAIL && P8 == 5) ? TM + TN : 0);
      static_assert(kAfter < 64, "vmcnt field");
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kAfter));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  });
}

template <int AF, int BF, bool BIAS, bool QUANT, int EPI, bool SPLIT, int BN>
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(Args p) {
  using SH = Shape<BN>;
  static_assert(!SPLIT || BN == kTile, "the split handoff's partial tiles are 256 x 256");
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st3[kStageBytes];
  __shared__ float lds_bias[kTile];
  uint8_t* const st[kStages] = {st0, st1, st2, st3};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave / SH::kWN, wn = wave % SH::kWN;

  int tile_id = blockIdx.x, ntiles = gridDim.x, split = 0;
  int tm, tn;
  if constexpr (SPLIT) {
    split = blockIdx.x % p.splits;
    tile_id = blockIdx.x / p.splits;
    ntiles = gridDim.x / p.splits;
    split_tile_of(tile_id, ntiles, p.splits, p.tiles_m, p.tiles_n, tm, tn);
  } else {
    tile_of(tile_id, ntiles, p.tiles_m, p.tiles_n, tm, tn);
  }
  const int64_t bz = blockIdx.y;
  const int m0 = tm * kTile, n0 = tn * BN;
  const int kb = p.K / 32;

  Pipe<AF, BF, BN> P;
  P.ca.init(p.a + bz * p.stride_a, m0, p.M, kTile, p.K, wave, lane, 0);
  P.cb.init(p.b + bz * p.stride_b, n0, p.N, BN, p.K, wave, lane, kBRegion);
  P.fa.init(p.a_s + bz * p.stride_as, m0, p.M, kb, wm * (kTile / SH::kWM), l32, h, 0);
  P.fb.init(p.b_s + bz * p.stride_bs, n0, p.N, kb, wn * (BN / SH::kWN), l32, h, kBRegion);

  // The tile's bias as fp32 in LDS for the epilogue (thread c: column c).
  const bool has_bias = BIAS && (EPI == kEpiPlain || p.bias != nullptr);
  uint32_t bias_bits = 0;
  if (has_bias)
    bias_bits = p.bias[bz * p.stride_bias + min(n0 + static_cast<int>(threadIdx.x), p.N - 1)];

  // Steps [k0, k0 + KT) of K (all of them unless SPLIT).  The launch guarantees K % 512 == 0
  // and, for SPLIT, ranges of a multiple of 8 steps starting on a multiple of 8.
  const int KT_all = p.K / 64;
  int k0 = 0, KT = KT_all;
  if constexpr (SPLIT) {
    k0 = split * (KT_all / p.splits);
    KT = KT_all / p.splits;
  }
  const int k_end = k0 + KT;
  v16f acc[SH::kTM][SH::kTN];
#pragma unroll
  for (int i = 0; i < SH::kTM; ++i)
#pragma unroll
    for (int j = 0; j < SH::kTN; ++j) acc[i][j] = v16f{};

  // Prologue: scale group 0, the copies of steps 0 and 1 and parts 0-2 of step 2's (the loop's
  // step 0 issues part 3, and scale group 1).
  using PP = Pipe<AF, BF, BN>;
  static_for<0, SH::kTM>([&](auto ic) { P.fa.template load_group<0, decltype(ic)::value>(k0, 0u); });
  static_for<0, SH::kTN>([&](auto ic) { P.fb.template load_group<0, decltype(ic)::value>(k0, 0u); });
  static_for<0, PP::kCp>([&](auto cc) { P.template copy<decltype(cc)::value>(st0, k0, 0u); });
  static_for<0, PP::kCp>([&](auto cc) {
    P.template copy<decltype(cc)::value>(st1, k0 + 1, past(k0 + 1, k_end));
  });
  static_for<0, PP::cut(3)>([&](auto cc) {
    P.template copy<decltype(cc)::value>(st2, k0 + 2, past(k0 + 2, k_end));
  });
  if (has_bias) lds_bias[threadIdx.x] = bf16_bits_to_f32(bias_bits);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(PP::kCp + PP::cut(3)));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  static_for<0, SH::kTM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    P.fa.template read<0, i, 0>(st0);
    if constexpr (byte_codes(AF)) P.fa.template read<1, i, 0>(st0);
  });
  static_for<0, SH::kTN>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    P.fb.template read<0, j, 0>(st0);
    if constexpr (byte_codes(BF)) P.fb.template read<1, j, 0>(st0);
  });
  P.fa.template take_scales<0, 0>();
  P.fb.template take_scales<0, 0>();
  static_for<0, SH::kTM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    P.opa[0][i] = P.fa.template decode<0, i, 0>();
  });
  static_for<0, SH::kTN>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    P.opb[0][j] = P.fb.template decode<0, j, 0>();
  });

  // The residual epilogue runs the range's last 8 steps apart (TAIL), to bring in the residual
  // tile while they run.
  constexpr bool kResTail = EPI == kEpiResidual && !SPLIT && !QUANT;
  ResTail<BN> R;
  R.on = false;
  if constexpr (kResTail) R.init(p, m0, n0, bz, wave, lane);
  int kl = 0;
  for (; kl < KT - (kResTail ? 8 : 0); kl += 8) {
    static_for<0, 8>([&](auto pc) {
      constexpr int p8 = decltype(pc)::value;
      mx_step<p8, false, AF, BF, BN>(P, R, st, acc, k0, kl + p8, k_end);
    });
  }
  if constexpr (kResTail) {
    static_for<0, 8>([&](auto pc) {
      constexpr int p8 = decltype(pc)::value;
      mx_step<p8, true, AF, BF, BN>(P, R, st, acc, k0, kl + p8, k_end);
    });
  }
  // The copies issued for steps past the range (or the residual's) may still be landing in the
  // stages the epilogue reuses.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);

  auto tile_row = [&](int r) -> uint8_t* {
    uint8_t* const base = r < 64 ? st0 : r < 128 ? st1 : r < 192 ? st2 : st3;
    return base + (r & 63) * (BN * 2);
  };
  finish_tile<AF, QUANT, EPI, SPLIT, kTile, BN, SH::kWM, SH::kWN>(p, acc, tile_row, lds_bias,
                                                                  has_bias, split, tile_id, m0,
                                                                  n0, bz, R.on);
}

template <int AF, int BF, bool BIAS, bool QUANT, int EPI, bool SPLIT, int BN = kTile>
hipError_t launch_mx(const Args& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_mx_kernel<AF, BF, BIAS, QUANT, EPI, SPLIT, BN>), grid, dim3(kThreads),
                     0, stream, p);
  return hipGetLastError();
}

template <int AF, int BF, int BN>
hipError_t launch_tiles_mx(const GemmProblem& g, const SplitPlan* plan, hipStream_t stream) {
  Args p{g.a, g.a_s, g.b, g.b_s, g.bias, g.c, g.M, g.N, g.K,
         (g.M + kTile - 1) / kTile, (g.N + BN - 1) / BN,
         g.stride_a, g.stride_as, g.stride_b, g.stride_bs, g.stride_bias, g.stride_c,
         g.q, g.qs, g.stride_q, g.stride_qs, g.residual, g.stride_res,
         nullptr, nullptr, 1};
  if constexpr (BN == kTile) {
    if (plan) {
      uint8_t* ws = static_cast<uint8_t*>(g.workspace);
      p.ws = reinterpret_cast<float*>(ws + plan->counter_bytes);
      p.counters = reinterpret_cast<uint32_t*>(ws);
      p.splits = plan->splits;
      dim3 grid(p.tiles_m * p.tiles_n * plan->splits, 1);
      return g.bias ? launch_mx<AF, BF, true, false, kEpiPlain, true>(p, grid, stream)
                    : launch_mx<AF, BF, false, false, kEpiPlain, true>(p, grid, stream);
    }
  }
  dim3 grid(p.tiles_m * p.tiles_n, g.batch);
  if constexpr (AF == kFp8 || AF == kFp4) {
    if (g.q) {
      if (g.epi == kEpiGelu)
        return launch_mx<AF, BF, true, true, kEpiGelu, false, BN>(p, grid, stream);
      return g.bias ? launch_mx<AF, BF, true, true, kEpiPlain, false, BN>(p, grid, stream)
                    : launch_mx<AF, BF, false, true, kEpiPlain, false, BN>(p, grid, stream);
    }
  }
  if (g.epi == kEpiResidual)
    return launch_mx<AF, BF, true, false, kEpiResidual, false, BN>(p, grid, stream);
  if (g.epi == kEpiGelu) return launch_mx<AF, BF, true, false, kEpiGelu, false, BN>(p, grid, stream);
  return g.bias ? launch_mx<AF, BF, true, false, kEpiPlain, false, BN>(p, grid, stream)
                : launch_mx<AF, BF, false, false, kEpiPlain, false, BN>(p, grid, stream);
}

template <int AF, int BF>
hipError_t launch_formats_mx(const GemmProblem& g, const SplitPlan* plan, int tile_n,
                             hipStream_t stream) {
  if (tile_n == 224 && !plan) return launch_tiles_mx<AF, BF, 224>(g, nullptr, stream);
  return launch_tiles_mx<AF, BF, kTile>(g, plan, stream);
}

}  // namespace

hipError_t launch_gemm_mx(int a_fmt, int b_fmt, const GemmProblem& p, const SplitPlan* plan,
                          int tile_n, hipStream_t stream) {
  if (tile_n != kTile && tile_n != 224) return hipErrorInvalidValue;
  if (a_fmt == kFp8 && b_fmt == kFp4) return launch_formats_mx<kFp8, kFp4>(p, plan, tile_n, stream);
  if (a_fmt == kFp8 && b_fmt == kFp8) return launch_formats_mx<kFp8, kFp8>(p, plan, tile_n, stream);
  if (a_fmt == kFp4 && b_fmt == kFp4) return launch_formats_mx<kFp4, kFp4>(p, plan, tile_n, stream);
  if (a_fmt == kBf8 && b_fmt == kFp8Rows)
    return launch_formats_mx<kBf8, kFp8Rows>(p, plan, tile_n, stream);
  return hipErrorInvalidValue;
}

}  // namespace mx
