/*
 * mx_c_driver -- drives the library's C ABI from C alone (no Python, no torch): device memory
 * from hipMalloc, every call through include/mx.h, one stream.  Test infrastructure: the GPU test
 * tests/test_gpu_c_driver.py writes the cases' inputs, runs this program once over all of them,
 * and checks its outputs against the oracle.
 *
 *   mx_c_driver DIR
 *
 * DIR/cases.txt holds one case per line:
 *   NAME KIND LAYOUT M N K BATCH
 *   KIND    fp8_fp4 | fp8_fp8 (A from bf16 activations through mx_act_quant) | fp4_fp4 (A given)
 *   LAYOUT  plain | bias | batched (distinct operands per batch, with bias) | broadcast (B, its
 *           scales and the bias shared by every batch: stride 0)
 * and DIR/NAME/ its inputs, raw little-endian arrays: x.bin (bf16, the activations) or a.bin +
 * a_s.bin (FP4 A), b.bin, b_s.bin, and bias.bin for the layouts with a bias; for the batched
 * layouts every per-batch array is the batches back to back (broadcast: B, its scales and the
 * bias once).  The program writes DIR/NAME/c.bin (bf16 output) and, when A comes from
 * activations, q.bin and s.bin (act_quant's codes and scale bytes).
 * Exit status 0 when every call returned MX_OK, else 1 with the failing call named on stderr.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mx.h"

static int fail(const char* what, const char* name, int st) {
  fprintf(stderr, "%s: %s failed: %d (%s)\n", name, what, st, mx_status_str(st));
  return 1;
}

static void* read_file(const char* dir, const char* name, const char* file, size_t want) {
  char path[1024];
  snprintf(path, sizeof path, "%s/%s/%s", dir, name, file);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return NULL;
  }
  void* buf = malloc(want ? want : 1);
  size_t got = fread(buf, 1, want, f);
  fclose(f);
  if (got != want) {
    fprintf(stderr, "%s: %zu bytes, expected %zu\n", path, got, want);
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* dir, const char* name, const char* file, const void* p, size_t n) {
  char path[1024];
  snprintf(path, sizeof path, "%s/%s/%s", dir, name, file);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = fwrite(p, 1, n, f);
  fclose(f);
  return put == n ? 0 : 1;
}

/* host bytes -> new device buffer (NULL on failure) */
static void* to_device(const void* host, size_t n) {
  void* d = NULL;
  if (hipMalloc(&d, n ? n : 16) != hipSuccess) return NULL;
  if (n && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) {
    hipFree(d);
    return NULL;
  }
  return d;
}

static int run_case(const char* dir, const char* name, const char* kind, const char* layout,
                    int64_t M, int64_t N, int64_t K, int64_t batch, hipStream_t st) {
  const int acts = strcmp(kind, "fp4_fp4") != 0;
  const int fp8w = strcmp(kind, "fp8_fp8") == 0;
  const int batched = strcmp(layout, "batched") == 0 || strcmp(layout, "broadcast") == 0;
  const int shared_b = strcmp(layout, "broadcast") == 0;
  const int has_bias = strcmp(layout, "plain") != 0;
  const int64_t nb = batched ? batch : 1;
  const int64_t kb = K / 32;
  /* per-batch element counts (bytes for codes and scales, bf16 elements for x, bias, c) */
  const int64_t n_a = acts ? M * K : M * (K / 2), n_as = M * kb;
  const int64_t n_b = fp8w ? N * K : N * (K / 2);
  const int64_t n_bs = fp8w ? ((N + 31) / 32) * kb : N * kb;
  const int64_t n_c = M * N;
  const int64_t nbb = shared_b ? 1 : nb;        /* batches held by B, its scales and the bias */
  int rc = 1;
  void *h_x = NULL, *h_a = NULL, *h_as = NULL, *h_b = NULL, *h_bs = NULL, *h_bias = NULL;
  void *d_x = NULL, *d_a = NULL, *d_as = NULL, *d_b = NULL, *d_bs = NULL, *d_bias = NULL,
       *d_c = NULL;
  void *h_c = NULL, *h_q = NULL, *h_s = NULL;

  if (acts) {
    h_x = read_file(dir, name, "x.bin", (size_t)(nb * M * K * 2));
    if (!h_x) goto done;
  } else {
    h_a = read_file(dir, name, "a.bin", (size_t)(nb * n_a));
    h_as = read_file(dir, name, "a_s.bin", (size_t)(nb * n_as));
    if (!h_a || !h_as) goto done;
  }
  h_b = read_file(dir, name, "b.bin", (size_t)(nbb * n_b));
  h_bs = read_file(dir, name, "b_s.bin", (size_t)(nbb * n_bs));
  if (!h_b || !h_bs) goto done;
  if (has_bias) {
    h_bias = read_file(dir, name, "bias.bin", (size_t)(nbb * N * 2));
    if (!h_bias) goto done;
  }

  d_b = to_device(h_b, (size_t)(nbb * n_b));
  d_bs = to_device(h_bs, (size_t)(nbb * n_bs));
  if (has_bias) d_bias = to_device(h_bias, (size_t)(nbb * N * 2));
  if (hipMalloc(&d_c, (size_t)(nb * n_c * 2)) != hipSuccess || !d_b || !d_bs ||
      (has_bias && !d_bias)) {
    fprintf(stderr, "%s: device allocation failed\n", name);
    goto done;
  }
  if (acts) {
    d_x = to_device(h_x, (size_t)(nb * M * K * 2));
    if (!d_x || hipMalloc(&d_a, (size_t)(nb * n_a)) != hipSuccess ||
        hipMalloc(&d_as, (size_t)(nb * n_as)) != hipSuccess) {
      fprintf(stderr, "%s: device allocation failed\n", name);
      goto done;
    }
    int s = batched ? mx_act_quant_strided_batched(d_x, d_a, d_as, M, K, nb, M * K, n_a, n_as, st)
                    : mx_act_quant(d_x, d_a, d_as, M, K, st);
    if (s != MX_OK) { rc = fail("act_quant", name, s); goto done; }
  } else {
    d_a = to_device(h_a, (size_t)(nb * n_a));
    d_as = to_device(h_as, (size_t)(nb * n_as));
    if (!d_a || !d_as) { fprintf(stderr, "%s: device allocation failed\n", name); goto done; }
  }

  {
    const int64_t sb = shared_b ? 0 : n_b, sbs = shared_b ? 0 : n_bs, sbias = shared_b ? 0 : N;
    int s;
    if (!strcmp(kind, "fp8_fp4")) {
      if (batched)
        s = mx_gemm_fp8_fp4_bias_strided_batched(d_a, d_as, d_b, d_bs, d_bias, d_c, M, N, K, nb,
                                                 n_a, n_as, sb, sbs, sbias, n_c, st);
      else if (has_bias)
        s = mx_gemm_fp8_fp4_bias(d_a, d_as, d_b, d_bs, d_bias, d_c, M, N, K, st);
      else
        s = mx_gemm_fp8_fp4(d_a, d_as, d_b, d_bs, d_c, M, N, K, st);
    } else if (fp8w) {
      if (batched)
        s = mx_gemm_fp8_fp8_bias_strided_batched(d_a, d_as, d_b, d_bs, d_bias, d_c, M, N, K, nb,
                                                 n_a, n_as, sb, sbs, sbias, n_c, st);
      else if (has_bias)
        s = mx_gemm_fp8_fp8_bias(d_a, d_as, d_b, d_bs, d_bias, d_c, M, N, K, st);
      else
        s = mx_gemm_fp8_fp8(d_a, d_as, d_b, d_bs, d_c, M, N, K, st);
    } else {
      if (batched)
        s = mx_gemm_fp4_fp4_bias_strided_batched(d_a, d_as, d_b, d_bs, d_bias, d_c, M, N, K, nb,
                                                 n_a, n_as, sb, sbs, sbias, n_c, st);
      else if (has_bias)
        s = mx_gemm_fp4_fp4_bias(d_a, d_as, d_b, d_bs, d_bias, d_c, M, N, K, st);
      else
        s = mx_gemm_fp4_fp4(d_a, d_as, d_b, d_bs, d_c, M, N, K, st);
    }
    if (s != MX_OK) { rc = fail("gemm", name, s); goto done; }
  }
  if (hipStreamSynchronize(st) != hipSuccess) {
    fprintf(stderr, "%s: stream synchronization failed\n", name);
    goto done;
  }
  h_c = malloc((size_t)(nb * n_c * 2));
  if (hipMemcpy(h_c, d_c, (size_t)(nb * n_c * 2), hipMemcpyDeviceToHost) != hipSuccess ||
      write_file(dir, name, "c.bin", h_c, (size_t)(nb * n_c * 2))) {
    fprintf(stderr, "%s: output copy failed\n", name);
    goto done;
  }
  if (acts) {
    h_q = malloc((size_t)(nb * n_a));
    h_s = malloc((size_t)(nb * n_as));
    if (hipMemcpy(h_q, d_a, (size_t)(nb * n_a), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(h_s, d_as, (size_t)(nb * n_as), hipMemcpyDeviceToHost) != hipSuccess ||
        write_file(dir, name, "q.bin", h_q, (size_t)(nb * n_a)) ||
        write_file(dir, name, "s.bin", h_s, (size_t)(nb * n_as))) {
      fprintf(stderr, "%s: act_quant output copy failed\n", name);
      goto done;
    }
  }
  rc = 0;
done:
  free(h_x); free(h_a); free(h_as); free(h_b); free(h_bs); free(h_bias);
  free(h_c); free(h_q); free(h_s);
  hipFree(d_x); hipFree(d_a); hipFree(d_as); hipFree(d_b); hipFree(d_bs); hipFree(d_bias);
  hipFree(d_c);
  return rc;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  mx_caps caps;
  int s = mx_capability(&caps);
  if (s != MX_OK || !caps.available) {
    fprintf(stderr, "no gfx950 device (%d)\n", s);
    return 1;
  }
  char path[1024];
  snprintf(path, sizeof path, "%s/cases.txt", argv[1]);
  FILE* f = fopen(path, "r");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  hipStream_t st;
  if (hipStreamCreate(&st) != hipSuccess) {
    fclose(f);
    return 1;
  }
  char name[256], kind[32], layout[32];
  long long M, N, K, batch;
  int failures = 0, cases = 0;
  while (fscanf(f, "%255s %31s %31s %lld %lld %lld %lld", name, kind, layout, &M, &N, &K,
                &batch) == 7) {
    ++cases;
    if (run_case(argv[1], name, kind, layout, M, N, K, batch, st)) ++failures;
  }
  fclose(f);
  hipStreamDestroy(st);
  printf("%d cases, %d failed\n", cases, failures);
  return failures ? 1 : 0;
}
