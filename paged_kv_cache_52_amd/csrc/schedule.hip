// Plan kernel: one workgroup running the plan of a decode step (see
// plan_device.h).
#include "plan_device.h"

namespace pa {

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const PlanParams p) {
  plan_workgroup(p);
}

hipError_t launch_plan(const PlanParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
