// The plan kernel: the tick's work lists (the one-wave plan of pa_plan.h) in a
// launch of its own, for the attention call.
#include "pa_plan.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 64;   // one wave
constexpr int kCachedSeqs = 4096;  // sequence shapes kept in LDS between the passes

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(AttnArgs a, int* plan, int cap_dec,
                                                            int cap_pf, int TM) {
  __shared__ PlanLds<kCachedSeqs> sm;
  plan_wave(a, plan, cap_dec, cap_pf, TM, sm);
}

}  // namespace

hipError_t launch_plan(const AttnArgs& a, int* plan, int cap_dec, int cap_pf, int TM,
                       hipStream_t s) {
  profile_before("plan", s);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a, plan, cap_dec, cap_pf,
                     TM);
  profile_after(s);
  return hipGetLastError();
}

}  // namespace pa
