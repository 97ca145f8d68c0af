// stepq_k64.hip -- d = 64 kernels, the debug decode and the side-stream spin (see
// stepq_device.h), and the launch dispatcher.
#include "stepq_device.h"

namespace stepq {

namespace {
// Bounded spin on the side stream (used by the ordering test): returns after `cycles` clocks.
__global__ void k_spin(long long cycles) {
  const long long t0 = (long long)__builtin_readcyclecounter();
  while ((long long)__builtin_readcyclecounter() - t0 < cycles) {
    __builtin_amdgcn_s_sleep(2);
  }
}
}  // namespace

hipError_t launch_gdn128(Mode mode, const StepArgs& a, hipStream_t s);
hipError_t launch_kda128(Mode mode, const StepArgs& a, hipStream_t s);

hipError_t launch_step(int kind, Mode mode, const StepArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.P.D == 64)
    return kind == 0 ? dev::launch_kind<64, 0>(mode, a, s) : dev::launch_kind<64, 1>(mode, a, s);
  return kind == 0 ? launch_gdn128(mode, a, s) : launch_kda128(mode, a, s);
}

hipError_t launch_unpack(const DevPlan& P, const uint8_t* pool, int B, float* S, uint16_t* r,
                         uint16_t* c, int8_t* z, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const dim3 grid(B * P.H);
  if (P.D == 64) hipLaunchKernelGGL(dev::k_unpack<64>, grid, dim3(64), 0, s, P, pool, S, r, c, z);
  else hipLaunchKernelGGL(dev::k_unpack<128>, grid, dim3(128), 0, s, P, pool, S, r, c, z);
  return hipGetLastError();
}

hipError_t launch_spin(long long cycles, hipStream_t s) {
  hipLaunchKernelGGL(k_spin, dim3(1), dim3(1), 0, s, cycles);
  return hipGetLastError();
}

}  // namespace stepq
