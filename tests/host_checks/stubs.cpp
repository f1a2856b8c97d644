// Stand-ins for the kernel launchers, so the C-ABI host code can be built
// and run with host sanitizers on a machine without a GPU.  A call that
// gets this far returns hipErrorNotReady, which the entry points report as
// PA_ERR_HIP: the driver expects that only where every host check passes.
#include <hip/hip_runtime.h>

#include "pa_internal.hpp"

namespace pa {

hipError_t launch_scatter(const void*, const void*, const int32_t*, void*, void*, int64_t, int32_t,
                          hipStream_t) {
  return hipErrorNotReady;
}
hipError_t launch_scatter_fp8(const void*, const void*, const int32_t*, const float*,
                              const float*, void*, void*, int64_t, int32_t, int32_t,
                              hipStream_t) {
  return hipErrorNotReady;
}
hipError_t launch_scatter_paged(const void*, const void*, const int32_t*, const int32_t*,
                                const int32_t*, void*, void*, const float*, const float*, int32_t,
                                int64_t, int32_t, int32_t, int32_t, int32_t, bool, hipStream_t) {
  return hipErrorNotReady;
}
hipError_t launch_rotary_scatter(const RotaryArgs&, int, hipStream_t) { return hipErrorNotReady; }
hipError_t launch_seqlens_from_past(const int32_t*, const int32_t*, int32_t*, int32_t,
                                    hipStream_t) {
  return hipErrorNotReady;
}
hipError_t launch_plan(const PlanArgs&, hipStream_t) { return hipErrorNotReady; }
int attention_workers(int, int, int num_cus, bool) { return num_cus; }
hipError_t launch_attention(const AttnArgs&, int, int, int, hipStream_t, bool) {
  return hipErrorNotReady;
}
hipError_t launch_combine(const AttnArgs&, int, int, hipStream_t) { return hipErrorNotReady; }

}  // namespace pa
