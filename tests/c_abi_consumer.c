/*
 * A plain C consumer of the library's C ABI (include/attn.h): device buffers
 * from the HIP runtime, no Python and no torch.  It calls attn_fwd on fp32
 * inputs with Q = 0, where every score is equal, so output row i is the mean
 * of the V rows it sees (all N, or rows 0..i under the causal mask) and its
 * LSE is the log of their count -- a closed form checked on the host.  It
 * also checks the ABI version and one rejected call.  Exit status 0 on
 * success.  Built and run by tests/test_gpu_c_abi.py.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "attn.h"

#define CHECK_HIP(x)                                                    \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
      return 2;                                                         \
    }                                                                   \
  } while (0)

int main(void) {
  const int B = 1, H = 2, N = 300, d = 64;
  const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
  float *hk = malloc(n * sizeof(float)), *hv = malloc(n * sizeof(float));
  float *ho = malloc(n * sizeof(float)), *hl = malloc(rows * sizeof(float));
  if (!hk || !hv || !ho || !hl) return 2;
  unsigned s = 12345u;   /* a small LCG: values in [-1, 1) */
  for (size_t i = 0; i < n; ++i) {
    s = s * 1664525u + 1013904223u;
    hk[i] = (float)((s >> 8) * (1.0 / 8388608.0)) - 1.f;
    s = s * 1664525u + 1013904223u;
    hv[i] = (float)((s >> 8) * (1.0 / 8388608.0)) - 1.f;
  }
  if (attn_abi_version() != ATTN_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", attn_abi_version(), ATTN_ABI_VERSION);
    return 1;
  }
  void *q, *k, *v, *o;
  float* lse;
  CHECK_HIP(hipMalloc(&q, n * sizeof(float)));
  CHECK_HIP(hipMalloc(&k, n * sizeof(float)));
  CHECK_HIP(hipMalloc(&v, n * sizeof(float)));
  CHECK_HIP(hipMalloc(&o, n * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&lse, rows * sizeof(float)));
  CHECK_HIP(hipMemset(q, 0, n * sizeof(float)));
  CHECK_HIP(hipMemcpy(k, hk, n * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv, n * sizeof(float), hipMemcpyHostToDevice));

  /* a head dimension the library does not implement: rejected before any HIP call */
  if (attn_fwd(ATTN_F32, B, H, N, 96, q, k, v, NULL, o, lse, 0.125f, 0, NULL) != ATTN_ERR_UNSUPPORTED) {
    fprintf(stderr, "d = 96 was not rejected\n");
    return 1;
  }
  for (int causal = 0; causal <= 1; ++causal) {
    int st = attn_fwd(ATTN_F32, B, H, N, d, q, k, v, NULL, o, lse, 0.125f, causal, NULL);
    if (st != ATTN_OK) {
      fprintf(stderr, "attn_fwd: %s: %s\n", attn_status_string(st), attn_last_error());
      return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(ho, o, n * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hl, lse, rows * sizeof(float), hipMemcpyDeviceToHost));
    double worst_o = 0.0, worst_l = 0.0;
    for (int bh = 0; bh < B * H; ++bh) {
      double acc[256] = {0.0};
      for (int i = 0; i < N; ++i) {
        const int count = causal ? i + 1 : N;
        /* running column sums of V over the rows row i sees */
        if (causal || i == 0) {
          const int from = causal ? i : 0, to = causal ? i + 1 : N;
          for (int j = from; j < to; ++j)
            for (int c = 0; c < d; ++c) acc[c] += hv[((size_t)bh * N + j) * d + c];
        }
        for (int c = 0; c < d; ++c) {
          const double e = fabs(ho[((size_t)bh * N + i) * d + c] - acc[c] / count);
          if (e > worst_o) worst_o = e;
        }
        const double el = fabs(hl[(size_t)bh * N + i] - log((double)count));
        if (el > worst_l) worst_l = el;
      }
    }
    printf("causal=%d: max |O - mean of visible V| %.3e, max |LSE - ln(count)| %.3e\n", causal, worst_o, worst_l);
    if (!(worst_o <= 1e-5) || !(worst_l <= 1e-5)) return 1;
  }
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(o);
  hipFree(lse);
  free(hk);
  free(hv);
  free(ho);
  free(hl);
  printf("ok\n");
  return 0;
}
