// Internal interface between the C-ABI layer (mx_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdint>

namespace mx {

// Operand encodings, numbered as the scaled f8f6f4 MFMA's format fields number them.
// kBf8 is E5M2 (backward gradients).  kFp8Rows is not an MFMA format: E4M3 codes whose E8M0
// scales run per row and 32 K (as activations'), where a kFp8 weight has 32x32 block scales; the
// backward GEMMs read transposed operands in that layout.
enum OperandFmt : int { kFp8 = 0, kBf8 = 1, kFp4 = 4, kFp8Rows = 8 };

// One code byte per value (E4M3 or E5M2), against packed E2M1.
constexpr bool byte_codes(int fmt) { return fmt != kFp4; }

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
  void* workspace = nullptr;            // split-K workspace (plan_split), or nullptr: no split
};

// Split-K plan of the tiled kernel for problems with fewer 256x256 output tiles than the 256 CUs
// of an MI355X and a long K (large down-projections): K is cut into two equal ranges of 64-wide
// steps, each range of each tile is one workgroup, and the first workgroup to finish a tile
// publishes its fp32 partial tile for the second, which adds it to its own.  Only single
// problems (batch 1) with 65..128 tiles (where the unsplit launch needs two or more waves of
// 128x128 tiles) and at least 40 steps per range: elsewhere the partial tiles' traffic (256 KB
// written and read per tile, through one CU) cost more than the idle CUs did (measured).  The
// plan depends on the shape alone, so the workspace size a caller asks for is the one the launch
// uses.  Workspace: `counter_bytes` holding a counter and a ready flag per tile (zero between
// calls), then one partial tile of 256 * 256 fp32 per tile.
struct SplitPlan {
  int splits = 1;
  int64_t counter_bytes = 0;
  int64_t bytes = 0;
};
constexpr int64_t kSplitTargetCUs = 256;
constexpr int64_t kMinSplitTiles = 65;
constexpr int64_t kMinStepsPerSplit = 40;
constexpr int64_t kSplitTileBytes = 256 * 256 * 4;

inline SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int64_t batch) {
  SplitPlan p;
  if (batch != 1 || M <= 0 || N <= 0 || K <= 0) return p;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t steps = (K + 63) / 64;
  if (2 * tiles > kSplitTargetCUs || tiles < kMinSplitTiles || steps < 2 * kMinStepsPerSplit)
    return p;
  p.splits = 2;
  p.counter_bytes = (tiles * 8 + 255) / 256 * 256;
  p.bytes = p.counter_bytes + tiles * kSplitTileBytes;
  return p;
}

struct DeviceInfo {
  int device;
  int cu_count;
  bool gfx950;
};

// Cached per-device properties of the calling thread's current device (false: no device).
bool current_device(DeviceInfo* info);

// fmt: kFp8 (E4M3 codes [M, K]), kFp4 (packed E2M1 [M, K/2]) or kBf8 (E5M2 codes [M, K], rounded
// to nearest even, or stochastically with `seed` when `stochastic`); scales E8M0 [M, K/32].
hipError_t launch_act_quant(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t M, int64_t K,
                            int64_t batch, int64_t stride_x, int64_t stride_q, int64_t stride_s,
                            hipStream_t stream, int fmt = kFp8, bool stochastic = false,
                            uint64_t seed = 0);

// Quantize-transpose: bf16 x [R, C] -> codes [C, R] + E8M0 [C, R/32] (blocks along R), E4M3 with
// act_quant's rule (fmt kFp8) or E5M2 with the gradient rule (fmt kBf8, RNE or stochastic).
// R % 32 == 0, C % 8 == 0, x and q 16-byte aligned.
hipError_t launch_quant_transpose(const uint16_t* x, uint8_t* q, uint8_t* s, int64_t R, int64_t C,
                                  hipStream_t stream, int fmt, bool stochastic, uint64_t seed);

// FP8-operand kinds: exact bf16 decode + bf16 MFMA (gemm_bf16.hip).
hipError_t launch_gemm_bf16(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                            hipStream_t stream);
// The same GEMMs on 256 x tile_n tiles (tile_n 256 or 224) with one wavefront per SIMD and
// operands staged raw into LDS by direct-to-LDS loads (gemm_mx.hip); `plan` non-null: split-K
// with p.workspace (256 x 256 tiles only).  It runs K in loop iterations of 8 steps of 64 (and
// reads scale bytes 4 steps at a time with 8-byte loads), so it takes K % 512 == 0, and for a
// split, ranges of a multiple of 8 steps.
inline bool mx_kernel_takes(int64_t K, int splits) {
  return K > 0 && K % 512 == 0 && ((K / 64) % (8 * splits)) == 0;
}
hipError_t launch_gemm_mx(int a_fmt, int b_fmt, const GemmProblem& p, const SplitPlan* plan,
                          int tile_n, hipStream_t stream);

// GEMM kernel for problems with few output tiles and a short K (gemm_small.hip): 64 x 64 tiles
// whose whole K of operand codes is copied into LDS at the start, in chunks of 256, at most four.
inline bool small_kernel_takes(int64_t K) { return K > 0 && K % 256 == 0 && K <= 1024; }
hipError_t launch_gemm_small(int a_fmt, int b_fmt, const GemmProblem& p, hipStream_t stream);

// Output tile width for that kernel: 224 where the problem's tiles of 256 x 224 fill the CUs'
// waves enough better than 256 x 256 tiles do to finish sooner, counting a wave of the narrower
// tiles as 224/256 of a wave of the wider (e.g. 4096 x 7168: 448 tiles of 256 x 256 take two
// waves of 256 CUs with the second one 3/4 full; 512 tiles of 256 x 224 take two full waves of
// 7/8 the work each); 256 otherwise.
inline int mx_tile_n(int64_t M, int64_t N, int64_t batch, int64_t cus) {
  auto waves = [&](int64_t bn) {
    const int64_t tiles = ((M + 255) / 256) * ((N + bn - 1) / bn) * batch;
    return (tiles + cus - 1) / cus;
  };
  return waves(224) * 224 < waves(256) * 256 ? 224 : 256;
}
// Both operands MXFP4 on the scaled f8f6f4 MFMA (gemm_fp4.hip).
hipError_t launch_gemm_fp4_mfma(const GemmProblem& p, int cus, hipStream_t stream);

// The split GEMM of p on this library's fixed device array instead of p.workspace (which it
// ignores), for callers that cannot allocate (gemm_scratch.hip); no_alloc_scratch_bytes() is the
// array's size.
hipError_t launch_gemm_no_alloc(int a_fmt, int b_fmt, GemmProblem p, const DeviceInfo& dev,
                                hipStream_t stream);
int64_t no_alloc_scratch_bytes();

// Picks the kernel for a problem.
hipError_t launch_gemm(int a_fmt, int b_fmt, const GemmProblem& p, const DeviceInfo& dev,
                       hipStream_t stream);

}  // namespace mx
