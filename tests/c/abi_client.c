/*
 * A plain C99 client of libstepq.so (include/stepq.h), with device memory from the HIP runtime
 * API and nothing else: no Python, no torch.  For a GDN plan (6-bit, 4-bit and FP16 pivot heads)
 * and a KDA plan (per-row widths 2/4/6/8, some FP16 pivot rows), both fused and split:
 *   1. encode a deterministic fp32 state and decode it back (stepq_unpack_debug);
 *   2. run an identity step (alpha = 1, beta = 0): A_t = I, so the readout must be S_hat^T q of
 *      the decoded state (checked per tile in binary64, relative L2 <= 1e-5);
 *   3. run a regular step and check the readout is finite and the status word stays clear.
 * Prints one line per plan and "c-abi: ok"; exits 0 on success, 1 on a failed check, 2 without
 * a GPU.  Built by __graft_entry__.build() with gcc against the in-tree library.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "stepq.h"

#define CHECK_HIP(x)                                                                 \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                       \
    }                                                                                \
  } while (0)
#define CHECK_SQ(x)                                                                  \
  do {                                                                               \
    int r_ = (x);                                                                    \
    if (r_ != STEPQ_OK) {                                                            \
      fprintf(stderr, "%s:%d %s -> %d: %s\n", __FILE__, __LINE__, #x, r_, stepq_last_error()); \
      exit(1);                                                                       \
    }                                                                                \
  } while (0)

/* deterministic uniform numbers in [-1, 1) (64-bit LCG, top 24 bits) */
static uint64_t g_state = 0x2545F4914F6CDD1Dull;
static float urand(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((double)(g_state >> 40) / 8388608.0 - 1.0);
}

static float* dev_copy(const float* h, size_t n) {
  float* d = NULL;
  CHECK_HIP(hipMalloc((void**)&d, n * sizeof(float)));
  CHECK_HIP(hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice));
  return d;
}

static int run_plan(int kind, int mode) {
  const int H = 3, D = 128, B = 2, T = B * H;
  const size_t nS = (size_t)T * D * D, nv = (size_t)T * D;
  const size_t na = kind == STEPQ_KIND_KDA ? nv : (size_t)T;
  int8_t bits[3 * 128];
  uint8_t piv[3 * 128];
  float om[3 * 128];
  for (int h = 0; h < H; h++)
    for (int i = 0; i < D; i++) {
      const int r = h * D + i;
      om[r] = 1.0f + 0.125f * (float)((r * 7) % 11);
      if (kind == STEPQ_KIND_GDN) {
        bits[r] = (int8_t)(h == 1 ? 4 : 6);
        piv[r] = (uint8_t)(h == 2);
      } else {
        bits[r] = (int8_t)(2 + 2 * ((r * 5) % 4));
        piv[r] = (uint8_t)(r % 37 == 5);
      }
    }
  stepq_plan_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.kind = kind;
  desc.n_heads = H;
  desc.d_k = desc.d_v = D;
  desc.bits = bits;
  desc.pivot = piv;
  desc.omega = om;
  desc.mode = mode;
  desc.max_batch = B;
  desc.device = 0;
  desc.order = STEPQ_ORDER_DELTA_FIRST;
  stepq_plan_t plan = NULL;
  CHECK_SQ(stepq_plan_create(&desc, &plan));
  size_t bpr = 0;
  double bpv = 0.0;
  CHECK_SQ(stepq_pool_bytes(plan, &bpr, &bpv));

  float* hS = (float*)malloc(nS * sizeof(float));
  float* hSh = (float*)malloc(nS * sizeof(float));
  float* hq = (float*)malloc(nv * sizeof(float));
  float* hk = (float*)malloc(nv * sizeof(float));
  float* hv = (float*)malloc(nv * sizeof(float));
  float* ha = (float*)malloc(na * sizeof(float));
  float* hb = (float*)malloc((size_t)T * sizeof(float));
  float* ho = (float*)malloc(nv * sizeof(float));
  for (size_t i = 0; i < nS; i++) hS[i] = 0.25f * urand();
  for (size_t i = 0; i < nv; i++) {
    hq[i] = urand();
    hk[i] = urand() * 0.0883883f; /* |k| about 1 */
    hv[i] = urand();
  }
  for (size_t i = 0; i < na; i++) ha[i] = 1.0f;
  for (int t = 0; t < T; t++) hb[t] = 0.0f;

  void* pool = NULL;
  CHECK_HIP(hipMalloc(&pool, (size_t)B * bpr));
  float* dS = dev_copy(hS, nS);
  float *dq = dev_copy(hq, nv), *dk = dev_copy(hk, nv), *dv = dev_copy(hv, nv);
  float *da = dev_copy(ha, na), *db = dev_copy(hb, (size_t)T);
  float* dout = NULL;
  CHECK_HIP(hipMalloc((void**)&dout, nv * sizeof(float)));
  CHECK_SQ(stepq_encode_state(plan, dS, pool, B, NULL));
  CHECK_SQ(stepq_unpack_debug(plan, pool, B, dS, NULL, NULL, NULL, NULL)); /* S_hat into dS */
  CHECK_SQ(stepq_sync(plan));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(hSh, dS, nS * sizeof(float), hipMemcpyDeviceToHost));

  /* identity step: the readout is S_hat^T q */
  CHECK_SQ(stepq_decode_step(plan, pool, B, dq, dk, dv, da, db, dout, NULL));
  CHECK_SQ(stepq_sync(plan));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho, dout, nv * sizeof(float), hipMemcpyDeviceToHost));
  double worst = 0.0;
  for (int t = 0; t < T; t++) {
    double num = 0.0, den = 0.0;
    for (int j = 0; j < D; j++) {
      double o = 0.0;
      for (int i = 0; i < D; i++) o += (double)hq[(size_t)t * D + i] * hSh[((size_t)t * D + i) * D + j];
      const double dlt = (double)ho[(size_t)t * D + j] - o;
      num += dlt * dlt;
      den += o * o;
    }
    const double rel = sqrt(num / (den > 0.0 ? den : 1.0));
    if (rel > worst) worst = rel;
  }

  /* a regular step */
  for (size_t i = 0; i < na; i++) ha[i] = 0.9f + 0.1f * fabsf(urand());
  for (int t = 0; t < T; t++) hb[t] = 0.5f + 0.25f * urand();
  CHECK_HIP(hipMemcpy(da, ha, na * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(db, hb, (size_t)T * sizeof(float), hipMemcpyHostToDevice));
  CHECK_SQ(stepq_decode_step(plan, pool, B, dq, dk, dv, da, db, dout, NULL));
  CHECK_SQ(stepq_sync(plan));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho, dout, nv * sizeof(float), hipMemcpyDeviceToHost));
  int finite = 1;
  for (size_t i = 0; i < nv; i++) finite &= isfinite(ho[i]) ? 1 : 0;
  uint32_t flags = 0;
  CHECK_SQ(stepq_get_status(plan, &flags, 1));

  printf("c-abi: %s %s: %zu bytes/request (%.3f bits/value), identity-step readout rel L2 %.2e, "
         "finite %d, status %u\n", kind == STEPQ_KIND_GDN ? "GDN" : "KDA",
         mode == STEPQ_MODE_FUSED ? "fused" : "split", bpr, bpv, worst, finite, flags);
  CHECK_SQ(stepq_plan_destroy(plan));
  hipFree(pool); hipFree(dS); hipFree(dq); hipFree(dk); hipFree(dv); hipFree(da); hipFree(db);
  hipFree(dout);
  free(hS); free(hSh); free(hq); free(hk); free(hv); free(ha); free(hb); free(ho);
  return worst <= 1e-5 && finite && flags == 0;
}

int main(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    fprintf(stderr, "c-abi: no GPU\n");
    return 2;
  }
  int ok = 1;
  ok &= run_plan(STEPQ_KIND_GDN, STEPQ_MODE_FUSED);
  ok &= run_plan(STEPQ_KIND_GDN, STEPQ_MODE_SPLIT);
  ok &= run_plan(STEPQ_KIND_KDA, STEPQ_MODE_FUSED);
  ok &= run_plan(STEPQ_KIND_KDA, STEPQ_MODE_SPLIT);
  printf("c-abi: %s\n", ok ? "ok" : "FAILED");
  return ok ? 0 : 1;
}
