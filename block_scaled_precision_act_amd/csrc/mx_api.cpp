// C ABI of the gfx950 microscaling library (declared in include/mx.h).
//
// Every entry point validates its arguments on the host first and returns a status code
// without touching HIP when they are wrong (the guards follow the "hip_quant PKG-INFO" page's
// memory-safety list: null pointers, narrowing of 64-bit sizes, grid limits, empty problems
// returning before a zero-sized launch).  Only then does it look up the current device and
// enqueue one kernel on the caller's stream.
#include "../../include/mx.h"
#include "mx_internal.h"

#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace mx {
namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxMatrixElems = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxBatch = 65535;

struct DeviceCache {
  std::once_flag once[kMaxDevices];
  DeviceInfo info[kMaxDevices];
  char arch[kMaxDevices][64];
};

DeviceCache& cache() {
  static DeviceCache c;
  return c;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool current_device(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return false;
  }
  DeviceCache& c = cache();
  std::call_once(c.once[dev], [&] {
    hipDeviceProp_t prop;
    DeviceInfo& d = c.info[dev];
    d.device = dev;
    d.cu_count = 0;
    d.gfx950 = false;
    c.arch[dev][0] = '\0';
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      d.cu_count = prop.multiProcessorCount;
      std::snprintf(c.arch[dev], sizeof(c.arch[dev]), "%s", prop.gcnArchName);
      d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    } else {
      (void)hipGetLastError();
    }
  });
  *out = c.info[dev];
  return true;
}

}  // namespace mx

using mx::DeviceInfo;
using mx::GemmProblem;

namespace {

int device_status(DeviceInfo* dev) {
  if (!mx::current_device(dev)) return MX_ERR_DEVICE;
  return dev->gfx950 ? MX_OK : MX_ERR_DEVICE;
}

int check_k(int64_t K) { return (K > 0 && K % 32 == 0) ? MX_OK : MX_ERR_SHAPE; }

int validate_act_quant(const void* x, void* q, void* s, int64_t M, int64_t K, int64_t batch,
                       int64_t sx, int64_t sq, int64_t ss) {
  if (check_k(K) != MX_OK || M < 0 || batch < 0) return MX_ERR_SHAPE;
  if (M > 0 && (M > mx::kMaxMatrixElems / K)) return MX_ERR_SHAPE;
  if (batch > mx::kMaxBatch) return MX_ERR_SHAPE;
  if (sx < 0 || sq < 0 || ss < 0) return MX_ERR_STRIDE;
  if (batch > 1 && (sq == 0 || ss == 0)) return MX_ERR_STRIDE;
  if (M == 0 || batch == 0) return MX_OK;
  if (!x || !q || !s) return MX_ERR_NULL;
  if (!mx::aligned16(x) || !mx::aligned16(q)) return MX_ERR_ALIGN;
  if ((sx * 2) % 16 != 0 || sq % 16 != 0) return MX_ERR_ALIGN;
  return MX_OK;
}

int act_quant_impl(const void* x, void* q, void* s, int64_t M, int64_t K, int64_t batch,
                   int64_t sx, int64_t sq, int64_t ss, void* stream, int fmt = mx::kFp8,
                   bool stochastic = false, uint64_t seed = 0) {
  int st = validate_act_quant(x, q, s, M, K, batch, sx, sq, ss);
  if (st != MX_OK || M == 0 || batch == 0) return st;
  DeviceInfo dev;
  if ((st = device_status(&dev)) != MX_OK) return st;
  hipError_t e = mx::launch_act_quant(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q),
                                      static_cast<uint8_t*>(s), M, K, batch, sx, sq, ss,
                                      static_cast<hipStream_t>(stream), fmt, stochastic, seed);
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

int quant_transpose_impl(const void* x, void* q, void* s, int64_t R, int64_t C, void* stream,
                         int fmt, bool stochastic, uint64_t seed) {
  if (R < 0 || C < 0 || R % 32 != 0 || C % 8 != 0) return MX_ERR_SHAPE;
  if (R > 0 && C > mx::kMaxMatrixElems / R) return MX_ERR_SHAPE;
  if (R == 0 || C == 0) return MX_OK;
  if (!x || !q || !s) return MX_ERR_NULL;
  if (!mx::aligned16(x) || !mx::aligned16(q)) return MX_ERR_ALIGN;
  int st;
  DeviceInfo dev;
  if ((st = device_status(&dev)) != MX_OK) return st;
  hipError_t e = mx::launch_quant_transpose(static_cast<const uint16_t*>(x),
                                            static_cast<uint8_t*>(q), static_cast<uint8_t*>(s),
                                            R, C, static_cast<hipStream_t>(stream), fmt,
                                            stochastic, seed);
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

struct GemmCall {
  int a_fmt, b_fmt;
  const void *a, *a_s, *b, *b_s, *bias;
  void* c;
  int64_t M, N, K, batch;
  int64_t sa, sas, sb, sbs, sbias, sc;
  bool needs_bias;
  // Quantized output (instead of c): E4M3 codes [M, N] and E8M0 bytes [M, N/32].
  bool quant = false;
  void* q = nullptr;
  void* qs = nullptr;
  int64_t sq = 0, sqs = 0;
  // Epilogue (bf16 output only): mx::kEpiResidual adds res [M, N]; mx::kEpiGelu applies GELU.
  int epi = mx::kEpiPlain;
  const void* res = nullptr;
  int64_t sres = 0;
  // Split-K workspace (the _splitk entry points).
  bool splitk = false;
  void* ws = nullptr;
  int64_t ws_bytes = 0;
  // Split-K on the library's own device array (the _splitk_noalloc entry point).
  bool no_alloc = false;
};

int validate_gemm(const GemmCall& g) {
  if (check_k(g.K) != MX_OK || g.M < 0 || g.N < 0 || g.batch < 0) return MX_ERR_SHAPE;
  if (g.batch > mx::kMaxBatch) return MX_ERR_SHAPE;
  if (g.M > 0 && g.M > mx::kMaxMatrixElems / g.K) return MX_ERR_SHAPE;
  if (g.N > 0 && g.N > mx::kMaxMatrixElems / g.K) return MX_ERR_SHAPE;
  if (g.M > 0 && g.N > 0 && g.M > mx::kMaxMatrixElems / g.N) return MX_ERR_SHAPE;
  if (g.quant && g.N % 32 != 0) return MX_ERR_SHAPE;
  if (g.sa < 0 || g.sas < 0 || g.sb < 0 || g.sbs < 0 || g.sbias < 0 || g.sc < 0 || g.sq < 0 ||
      g.sqs < 0 || g.sres < 0)
    return MX_ERR_STRIDE;
  if (g.batch > 1 && (g.quant ? (g.sq == 0 || g.sqs == 0) : g.sc == 0)) return MX_ERR_STRIDE;
  if (g.M == 0 || g.N == 0 || g.batch == 0) return MX_OK;
  if (!g.a || !g.a_s || !g.b || !g.b_s) return MX_ERR_NULL;
  if (g.quant ? (!g.q || !g.qs) : !g.c) return MX_ERR_NULL;
  if (g.needs_bias && !g.bias) return MX_ERR_NULL;
  if (g.splitk) {
    const mx::SplitPlan plan = mx::plan_split(g.M, g.N, g.K, g.batch);
    if (plan.splits > 1 && (!g.ws || g.ws_bytes < plan.bytes ||
                            (reinterpret_cast<uintptr_t>(g.ws) & 255u) != 0))
      return MX_ERR_WORKSPACE;
  }
  if (g.no_alloc) {
    const mx::SplitPlan plan = mx::plan_split(g.M, g.N, g.K, g.batch);
    if (plan.splits > 1 && plan.bytes > mx::no_alloc_scratch_bytes()) return MX_ERR_WORKSPACE;
  }
  if (g.epi == mx::kEpiResidual && !g.res) return MX_ERR_NULL;
  if (!mx::aligned16(g.a) || !mx::aligned16(g.b)) return MX_ERR_ALIGN;
  if (g.sa % 16 != 0 || g.sb % 16 != 0) return MX_ERR_ALIGN;
  if (g.quant && (!mx::aligned16(g.q) || g.sq % 16 != 0)) return MX_ERR_ALIGN;
  return MX_OK;
}

int gemm_impl(const GemmCall& g, void* stream) {
  int st = validate_gemm(g);
  if (st != MX_OK || g.M == 0 || g.N == 0 || g.batch == 0) return st;
  DeviceInfo dev;
  if ((st = device_status(&dev)) != MX_OK) return st;
  GemmProblem p;
  p.a = static_cast<const uint8_t*>(g.a);
  p.a_s = static_cast<const uint8_t*>(g.a_s);
  p.b = static_cast<const uint8_t*>(g.b);
  p.b_s = static_cast<const uint8_t*>(g.b_s);
  p.bias = static_cast<const uint16_t*>(g.bias);
  p.c = static_cast<uint16_t*>(g.c);
  p.M = static_cast<int>(g.M);
  p.N = static_cast<int>(g.N);
  p.K = static_cast<int>(g.K);
  p.batch = static_cast<int>(g.batch);
  p.stride_a = g.sa;
  p.stride_as = g.sas;
  p.stride_b = g.sb;
  p.stride_bs = g.sbs;
  p.stride_bias = g.sbias;
  p.stride_c = g.sc;
  p.epi = g.epi;
  p.residual = static_cast<const uint16_t*>(g.res);
  p.stride_res = g.sres;
  if (g.splitk) p.workspace = g.ws;
  if (g.quant) {
    p.c = nullptr;
    p.q = static_cast<uint8_t*>(g.q);
    p.qs = static_cast<uint8_t*>(g.qs);
    p.stride_q = g.sq;
    p.stride_qs = g.sqs;
  }
  hipError_t e = g.no_alloc
      ? mx::launch_gemm_no_alloc(g.a_fmt, g.b_fmt, p, dev, static_cast<hipStream_t>(stream))
      : mx::launch_gemm(g.a_fmt, g.b_fmt, p, dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

GemmCall single(int af, int bf, const void* a, const void* a_s, const void* b, const void* b_s,
                const void* bias, void* c, int64_t M, int64_t N, int64_t K, bool needs_bias) {
  return GemmCall{af, bf, a, a_s, b, b_s, bias, c, M, N, K, 1, 0, 0, 0, 0, 0, 0, needs_bias};
}

GemmCall batched(int af, int bf, const void* a, const void* a_s, const void* b, const void* b_s,
                 const void* bias, void* c, int64_t M, int64_t N, int64_t K, int64_t batch,
                 int64_t sa, int64_t sas, int64_t sb, int64_t sbs, int64_t sbias, int64_t sc,
                 bool needs_bias) {
  return GemmCall{af, bf, a, a_s, b, b_s, bias, c, M, N, K, batch,
                  sa, sas, sb, sbs, sbias, sc, needs_bias};
}

GemmCall with_workspace(GemmCall g, void* ws, int64_t ws_bytes) {
  g.splitk = true;
  g.ws = ws;
  g.ws_bytes = ws_bytes;
  return g;
}

GemmCall with_epilogue(GemmCall g, int epi, const void* res, int64_t sres) {
  g.epi = epi;
  g.res = res;
  g.sres = sres;
  return g;
}

GemmCall quantized(int af, int bf, const void* a, const void* a_s, const void* b,
                   const void* b_s, const void* bias, void* q, void* qs, int64_t M, int64_t N,
                   int64_t K, int64_t batch, int64_t sa, int64_t sas, int64_t sb, int64_t sbs,
                   int64_t sbias, int64_t sq, int64_t sqs) {
  GemmCall g{af, bf, a, a_s, b, b_s, bias, nullptr, M, N, K, batch,
             sa, sas, sb, sbs, sbias, 0, false};
  g.quant = true;
  g.q = q;
  g.qs = qs;
  g.sq = sq;
  g.sqs = sqs;
  return g;
}

}  // namespace

extern "C" {

int mx_capability(mx_caps* caps) {
  if (!caps) return MX_ERR_NULL;
  std::memset(caps, 0, sizeof(*caps));
  caps->device = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    std::snprintf(caps->reason, sizeof(caps->reason), "no HIP device is visible");
    return MX_ERR_DEVICE;
  }
  DeviceInfo dev;
  if (!mx::current_device(&dev)) {
    std::snprintf(caps->reason, sizeof(caps->reason), "hipGetDevice failed");
    return MX_ERR_DEVICE;
  }
  caps->device = dev.device;
  caps->compute_units = dev.cu_count;
  std::snprintf(caps->arch, sizeof(caps->arch), "%s", mx::cache().arch[dev.device]);
  if (!dev.gfx950) {
    std::snprintf(caps->reason, sizeof(caps->reason),
                  "device %d is %s; these kernels are built for gfx950 only", dev.device,
                  caps->arch);
    return MX_ERR_DEVICE;
  }
  caps->available = 1;
  return MX_OK;
}

const char* mx_status_str(int status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 32; sizes >= 0 and within limits)";
    case MX_ERR_ALIGN: return "an operand pointer or batch stride is not 16-byte aligned";
    case MX_ERR_STRIDE: return "invalid stride (negative, or output stride 0 with batch > 1)";
    case MX_ERR_DEVICE: return "no gfx950 device is current";
    case MX_ERR_LAUNCH: return "kernel launch failed";
    case MX_ERR_WORKSPACE: return "split-K workspace missing, too small or not 256-byte aligned";
    default: return "unknown status";
  }
}

int mx_act_quant(const void* x, void* q, void* s, int64_t M, int64_t K, void* stream) {
  return act_quant_impl(x, q, s, M, K, 1, 0, 0, 0, stream);
}

int mx_act_quant_strided_batched(const void* x, void* q, void* s, int64_t M, int64_t K,
                                 int64_t batch, int64_t stride_x, int64_t stride_q,
                                 int64_t stride_s, void* stream) {
  return act_quant_impl(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream);
}

int mx_act_quant_fp4(const void* x, void* q, void* s, int64_t M, int64_t K, void* stream) {
  return act_quant_impl(x, q, s, M, K, 1, 0, 0, 0, stream, mx::kFp4);
}

int mx_act_quant_fp4_strided_batched(const void* x, void* q, void* s, int64_t M, int64_t K,
                                     int64_t batch, int64_t stride_x, int64_t stride_q,
                                     int64_t stride_s, void* stream) {
  return act_quant_impl(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream, mx::kFp4);
}

int mx_quant_e5m2(const void* x, void* q, void* s, int64_t M, int64_t K, int stochastic,
                  uint64_t seed, void* stream) {
  return act_quant_impl(x, q, s, M, K, 1, 0, 0, 0, stream, mx::kBf8, stochastic != 0, seed);
}

int mx_quant_e5m2_strided_batched(const void* x, void* q, void* s, int64_t M, int64_t K,
                                  int64_t batch, int64_t stride_x, int64_t stride_q,
                                  int64_t stride_s, int stochastic, uint64_t seed, void* stream) {
  return act_quant_impl(x, q, s, M, K, batch, stride_x, stride_q, stride_s, stream, mx::kBf8,
                        stochastic != 0, seed);
}

int mx_quant_transpose_e4m3(const void* x, void* q, void* s, int64_t R, int64_t C, void* stream) {
  return quant_transpose_impl(x, q, s, R, C, stream, mx::kFp8, false, 0);
}

int mx_quant_transpose_e5m2(const void* x, void* q, void* s, int64_t R, int64_t C, int stochastic,
                            uint64_t seed, void* stream) {
  return quant_transpose_impl(x, q, s, R, C, stream, mx::kBf8, stochastic != 0, seed);
}

int mx_gemm_e5m2_e4m3(const void* a, const void* a_s, const void* b, const void* b_s, void* c,
                      int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_impl(single(mx::kBf8, mx::kFp8Rows, a, a_s, b, b_s, nullptr, c, M, N, K, false),
                   stream);
}

int mx_gemm_e5m2_e4m3_splitk(const void* a, const void* a_s, const void* b, const void* b_s,
                             void* c, int64_t M, int64_t N, int64_t K, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return gemm_impl(with_workspace(single(mx::kBf8, mx::kFp8Rows, a, a_s, b, b_s, nullptr, c, M, N,
                                         K, false),
                                  workspace, workspace_bytes),
                   stream);
}

int mx_gemm_e5m2_e4m3_strided_batched(const void* a, const void* a_s, const void* b,
                                      const void* b_s, void* c, int64_t M, int64_t N, int64_t K,
                                      int64_t batch, int64_t sa, int64_t sas, int64_t sb,
                                      int64_t sbs, int64_t sc, void* stream) {
  return gemm_impl(batched(mx::kBf8, mx::kFp8Rows, a, a_s, b, b_s, nullptr, c, M, N, K, batch, sa,
                           sas, sb, sbs, 0, sc, false),
                   stream);
}

#define MX_GEMM_ENTRY_POINTS(NAME, AF, BF)                                                    \
  int mx_gemm_##NAME(const void* a, const void* a_s, const void* b, const void* b_s, void* c, \
                     int64_t M, int64_t N, int64_t K, void* stream) {                         \
    return gemm_impl(single(AF, BF, a, a_s, b, b_s, nullptr, c, M, N, K, false), stream);     \
  }                                                                                           \
  int mx_gemm_##NAME##_bias(const void* a, const void* a_s, const void* b, const void* b_s,   \
                            const void* bias, void* c, int64_t M, int64_t N, int64_t K,       \
                            void* stream) {                                                   \
    return gemm_impl(single(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, true), stream);         \
  }                                                                                           \
  int mx_gemm_##NAME##_strided_batched(const void* a, const void* a_s, const void* b,         \
                                       const void* b_s, void* c, int64_t M, int64_t N,        \
                                       int64_t K, int64_t batch, int64_t sa, int64_t sas,     \
                                       int64_t sb, int64_t sbs, int64_t sc, void* stream) {   \
    return gemm_impl(batched(AF, BF, a, a_s, b, b_s, nullptr, c, M, N, K, batch, sa, sas, sb, \
                             sbs, 0, sc, false),                                              \
                     stream);                                                                 \
  }                                                                                           \
  int mx_gemm_##NAME##_bias_strided_batched(                                                  \
      const void* a, const void* a_s, const void* b, const void* b_s, const void* bias,       \
      void* c, int64_t M, int64_t N, int64_t K, int64_t batch, int64_t sa, int64_t sas,       \
      int64_t sb, int64_t sbs, int64_t sbias, int64_t sc, void* stream) {                     \
    return gemm_impl(batched(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, batch, sa, sas, sb,    \
                             sbs, sbias, sc, true),                                           \
                     stream);                                                                 \
  }

MX_GEMM_ENTRY_POINTS(fp8_fp4, mx::kFp8, mx::kFp4)
MX_GEMM_ENTRY_POINTS(fp8_fp8, mx::kFp8, mx::kFp8)
MX_GEMM_ENTRY_POINTS(fp4_fp4, mx::kFp4, mx::kFp4)

#undef MX_GEMM_ENTRY_POINTS

#define MX_GEMM_QUANT_ENTRY_POINTS(NAME, AF, BF)                                              \
  int mx_gemm_##NAME##_quant(const void* a, const void* a_s, const void* b, const void* b_s,  \
                             const void* bias, void* q, void* q_s, int64_t M, int64_t N,      \
                             int64_t K, void* stream) {                                       \
    return gemm_impl(quantized(AF, BF, a, a_s, b, b_s, bias, q, q_s, M, N, K, 1, 0, 0, 0, 0,  \
                               0, 0, 0),                                                      \
                     stream);                                                                 \
  }                                                                                           \
  int mx_gemm_##NAME##_quant_strided_batched(                                                 \
      const void* a, const void* a_s, const void* b, const void* b_s, const void* bias,       \
      void* q, void* q_s, int64_t M, int64_t N, int64_t K, int64_t batch, int64_t sa,         \
      int64_t sas, int64_t sb, int64_t sbs, int64_t sbias, int64_t sq, int64_t sqs,           \
      void* stream) {                                                                         \
    return gemm_impl(quantized(AF, BF, a, a_s, b, b_s, bias, q, q_s, M, N, K, batch, sa, sas, \
                               sb, sbs, sbias, sq, sqs),                                      \
                     stream);                                                                 \
  }

MX_GEMM_QUANT_ENTRY_POINTS(fp8_fp4, mx::kFp8, mx::kFp4)
MX_GEMM_QUANT_ENTRY_POINTS(fp8_fp8, mx::kFp8, mx::kFp8)
MX_GEMM_QUANT_ENTRY_POINTS(fp4_fp4, mx::kFp4, mx::kFp4)

#undef MX_GEMM_QUANT_ENTRY_POINTS

// GELU before the quantized output (bias optional).
#define MX_GEMM_GELU_QUANT_ENTRY_POINTS(NAME, AF, BF)                                         \
  int mx_gemm_##NAME##_bias_gelu_quant(const void* a, const void* a_s, const void* b,         \
                                       const void* b_s, const void* bias, void* q, void* q_s, \
                                       int64_t M, int64_t N, int64_t K, void* stream) {       \
    return gemm_impl(with_epilogue(quantized(AF, BF, a, a_s, b, b_s, bias, q, q_s, M, N, K,   \
                                             1, 0, 0, 0, 0, 0, 0, 0),                         \
                                   mx::kEpiGelu, nullptr, 0),                                 \
                     stream);                                                                 \
  }                                                                                           \
  int mx_gemm_##NAME##_bias_gelu_quant_strided_batched(                                       \
      const void* a, const void* a_s, const void* b, const void* b_s, const void* bias,       \
      void* q, void* q_s, int64_t M, int64_t N, int64_t K, int64_t batch, int64_t sa,         \
      int64_t sas, int64_t sb, int64_t sbs, int64_t sbias, int64_t sq, int64_t sqs,           \
      void* stream) {                                                                         \
    return gemm_impl(with_epilogue(quantized(AF, BF, a, a_s, b, b_s, bias, q, q_s, M, N, K,   \
                                             batch, sa, sas, sb, sbs, sbias, sq, sqs),        \
                                   mx::kEpiGelu, nullptr, 0),                                 \
                     stream);                                                                 \
  }

MX_GEMM_GELU_QUANT_ENTRY_POINTS(fp8_fp4, mx::kFp8, mx::kFp4)
MX_GEMM_GELU_QUANT_ENTRY_POINTS(fp8_fp8, mx::kFp8, mx::kFp8)
MX_GEMM_GELU_QUANT_ENTRY_POINTS(fp4_fp4, mx::kFp4, mx::kFp4)

#undef MX_GEMM_GELU_QUANT_ENTRY_POINTS

// The bias is optional (NULL adds nothing) in the residual and GELU entry points.
#define MX_GEMM_EPILOGUE_ENTRY_POINTS(NAME, AF, BF)                                           \
  int mx_gemm_##NAME##_bias_residual(const void* a, const void* a_s, const void* b,           \
                                     const void* b_s, const void* bias, const void* residual, \
                                     void* c, int64_t M, int64_t N, int64_t K, void* stream) { \
    return gemm_impl(with_epilogue(single(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, false),   \
                                   mx::kEpiResidual, residual, 0),                            \
                     stream);                                                                 \
  }                                                                                           \
  int mx_gemm_##NAME##_bias_residual_strided_batched(                                         \
      const void* a, const void* a_s, const void* b, const void* b_s, const void* bias,       \
      const void* residual, void* c, int64_t M, int64_t N, int64_t K, int64_t batch,          \
      int64_t sa, int64_t sas, int64_t sb, int64_t sbs, int64_t sbias, int64_t sres,          \
      int64_t sc, void* stream) {                                                             \
    return gemm_impl(with_epilogue(batched(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, batch,   \
                                           sa, sas, sb, sbs, sbias, sc, false),               \
                                   mx::kEpiResidual, residual, sres),                         \
                     stream);                                                                 \
  }                                                                                           \
  int mx_gemm_##NAME##_bias_gelu(const void* a, const void* a_s, const void* b,               \
                                 const void* b_s, const void* bias, void* c, int64_t M,       \
                                 int64_t N, int64_t K, void* stream) {                        \
    return gemm_impl(with_epilogue(single(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, false),   \
                                   mx::kEpiGelu, nullptr, 0),                                 \
                     stream);                                                                 \
  }                                                                                           \
  int mx_gemm_##NAME##_bias_gelu_strided_batched(                                             \
      const void* a, const void* a_s, const void* b, const void* b_s, const void* bias,       \
      void* c, int64_t M, int64_t N, int64_t K, int64_t batch, int64_t sa, int64_t sas,       \
      int64_t sb, int64_t sbs, int64_t sbias, int64_t sc, void* stream) {                     \
    return gemm_impl(with_epilogue(batched(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, batch,   \
                                           sa, sas, sb, sbs, sbias, sc, false),               \
                                   mx::kEpiGelu, nullptr, 0),                                 \
                     stream);                                                                 \
  }

int64_t mx_gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (check_k(K) != MX_OK || M < 0 || N < 0) return 0;
  return mx::plan_split(M, N, K, 1).bytes;
}

#define MX_GEMM_SPLITK_ENTRY_POINT(NAME, AF, BF)                                              \
  int mx_gemm_##NAME##_splitk(const void* a, const void* a_s, const void* b, const void* b_s, \
                              const void* bias, void* c, int64_t M, int64_t N, int64_t K,     \
                              void* workspace, int64_t workspace_bytes, void* stream) {       \
    return gemm_impl(with_workspace(single(AF, BF, a, a_s, b, b_s, bias, c, M, N, K, false),  \
                                    workspace, workspace_bytes),                              \
                     stream);                                                                 \
  }

int mx_gemm_fp8_fp4_splitk_noalloc(const void* a, const void* a_s, const void* b,
                                   const void* b_s, const void* bias, void* c, int64_t M,
                                   int64_t N, int64_t K, void* stream) {
  GemmCall g = single(mx::kFp8, mx::kFp4, a, a_s, b, b_s, bias, c, M, N, K, false);
  g.no_alloc = true;
  return gemm_impl(g, stream);
}

MX_GEMM_SPLITK_ENTRY_POINT(fp8_fp4, mx::kFp8, mx::kFp4)
MX_GEMM_SPLITK_ENTRY_POINT(fp8_fp8, mx::kFp8, mx::kFp8)
MX_GEMM_SPLITK_ENTRY_POINT(fp4_fp4, mx::kFp4, mx::kFp4)

#undef MX_GEMM_SPLITK_ENTRY_POINT

MX_GEMM_EPILOGUE_ENTRY_POINTS(fp8_fp4, mx::kFp8, mx::kFp4)
MX_GEMM_EPILOGUE_ENTRY_POINTS(fp8_fp8, mx::kFp8, mx::kFp8)
MX_GEMM_EPILOGUE_ENTRY_POINTS(fp4_fp4, mx::kFp4, mx::kFp4)

#undef MX_GEMM_EPILOGUE_ENTRY_POINTS

}  // extern "C"
