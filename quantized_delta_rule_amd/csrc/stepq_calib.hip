// stepq_calib.hip -- calibration estimators on the device.
//
// Row impact (page: "STEPQuant" paper digest, vibe-research silicon-writer readme, Method 2):
// a quantization error E in the state reaches the next readout as (A_t^T q_t)^T E, so row i
// matters in proportion to omega_i = E[g_i^2] with g = A_t^T q_t.  For
// A_t = Diag(a)(I - beta k k^T):  g = a*q - beta k (k . (a*q));  for the other gate order,
// A_t = (I - beta k k^T) Diag(a):  g = a * (q - beta k (k . q)).
//
// One workgroup per head, one thread per key row.  Samples (requests) are taken in index order
// and each thread keeps its row's sum in binary64, so the result does not depend on scheduling.
#include <hip/hip_runtime.h>

#include "stepq_internal.h"

namespace stepq {
namespace {

template <int D>
__global__ __launch_bounds__(D) void k_row_impact(int kda, int order, int H, int B,
                                                  const float* q, const float* k,
                                                  const float* alpha, const float* beta,
                                                  double* acc) {
  __shared__ double red[D];
  const int h = blockIdx.x, i = threadIdx.x;
  double sum = 0.0;
  for (int b = 0; b < B; b++) {
    const long long t = (long long)b * H + h;
    const double a = kda ? (double)alpha[t * D + i] : (double)alpha[t];
    const double ki = (double)k[t * D + i], qi = (double)q[t * D + i];
    const double aq = a * qi;
    red[i] = ki * (order ? qi : aq);
    __syncthreads();
    for (int n = D / 2; n > 0; n >>= 1) {  // k . (a*q) or k . q: pairwise halving
      if (i < n) red[i] = red[i] + red[i + n];
      __syncthreads();
    }
    const double kx = red[0];
    __syncthreads();  // red is rewritten by the next sample
    const double s = (double)beta[t] * kx;
    const double g = order ? a * (qi - s * ki) : aq - s * ki;
    sum = sum + g * g;
  }
  acc[(long long)h * D + i] += sum;
}

}  // namespace

hipError_t launch_row_impact(int kind, int order, int H, int D, int B, const float* q,
                             const float* k, const float* alpha, const float* beta, double* acc,
                             hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (D == 64)
    hipLaunchKernelGGL(k_row_impact<64>, dim3(H), dim3(64), 0, s, kind, order, H, B, q, k, alpha,
                       beta, acc);
  else
    hipLaunchKernelGGL(k_row_impact<128>, dim3(H), dim3(128), 0, s, kind, order, H, B, q, k,
                       alpha, beta, acc);
  return hipGetLastError();
}

}  // namespace stepq
