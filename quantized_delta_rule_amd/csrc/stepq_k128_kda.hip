// stepq_k128_kda.hip -- d = 128 KDA kernels (see stepq_device.h).
#include "stepq_device.h"

namespace stepq {
hipError_t launch_kda128(Mode mode, const StepArgs& a, hipStream_t s) {
  return dev::launch_kind<128, 1>(mode, a, s);
}
}  // namespace stepq
