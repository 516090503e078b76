// The split-K FP8 x MXFP4 GEMM without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its per-tile counters, ready flags and partial tiles live in one fixed device
// array of this library instead: a 32 MB + 1 KB array that every GPU the library runs on holds
// until the process ends.  That covers the largest split plan (128 output tiles of 256 x 256:
// 1 KB of counters and flags, then one 256 KB fp32 partial tile per tile).
//
// Every call on a GPU shares that GPU's array, which keeps the last call's contents: calls that
// overlap on one GPU (concurrent streams) race and must not be made.  Each call first clears the
// counters and flags it will use with a small fill kernel on its stream (no memset node, so the
// call can be captured in a graph), then runs the split GEMM on the array.
#include "mx_internal.h"

#include <mutex>

namespace mx {
namespace {

constexpr int kMaxScratchDevices = 64;
constexpr int64_t kScratchCounterBytes = 1024;      // counter + flag per tile, up to 128 tiles
constexpr int64_t kScratchBytes = kScratchCounterBytes + 128 * kSplitTileBytes;

// In host code this name is a stand-in, not a device address: the device address of each GPU's
// copy comes from hipGetSymbolAddress (scratch_address below), and only that is ever used.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + static_cast<int>(threadIdx.x);
  if (i < n) p[i] = 0u;
}

struct ScratchAddresses {
  std::once_flag once[kMaxScratchDevices];
  void* ptr[kMaxScratchDevices] = {};
  hipError_t err[kMaxScratchDevices] = {};
};

ScratchAddresses& addresses() {
  static ScratchAddresses a;
  return a;
}

// Device address of the array on `device`, which must be the current device: looked up once per
// device (its first call here), with that device current.
hipError_t scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
  ScratchAddresses& a = addresses();
  std::call_once(a.once[device], [&] {
    void* p = nullptr;
    a.err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    a.ptr[device] = a.err[device] == hipSuccess ? p : nullptr;
  });
  *out = a.ptr[device];
  return a.err[device];
}

}  // namespace

int64_t no_alloc_scratch_bytes() { return kScratchBytes; }

hipError_t launch_gemm_no_alloc(int a_fmt, int b_fmt, GemmProblem p, const DeviceInfo& dev,
                                hipStream_t stream) {
  const SplitPlan plan = plan_split(p.M, p.N, p.K, p.batch);
  p.workspace = nullptr;
  if (plan.splits > 1) {
    if (plan.bytes > kScratchBytes || plan.counter_bytes > kScratchCounterBytes)
      return hipErrorInvalidValue;                   // the C ABI refuses this before we get here
    void* ws = nullptr;
    hipError_t e = scratch_address(dev.device, &ws);
    if (e != hipSuccess) return e;
    const int words = static_cast<int>(plan.counter_bytes / 4);
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    p.workspace = ws;
  }
  return launch_gemm(a_fmt, b_fmt, p, dev, stream);
}

}  // namespace mx
