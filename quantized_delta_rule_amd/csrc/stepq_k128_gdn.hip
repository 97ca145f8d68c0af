// stepq_k128_gdn.hip -- d = 128 GDN kernels (see stepq_device.h).
#include "stepq_device.h"

namespace stepq {
hipError_t launch_gdn128(Mode mode, const StepArgs& a, hipStream_t s) {
  return dev::launch_kind<128, 0>(mode, a, s);
}
}  // namespace stepq
