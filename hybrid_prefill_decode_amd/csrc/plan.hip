// Stand-alone launch of the plan (the layer step builds it inside its first prep pass instead;
// plan_core.h describes the lists).
#include "plan_core.h"

namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* __restrict__ q_start,
                                                        const int32_t* __restrict__ num_cached,
                                                        int num_seqs,
                                                        const int32_t* __restrict__ table,
                                                        int max_blocks, hl::Plan p) {
  __shared__ hl::plan::Shared<kThreads> sh;
  hl::plan::build<kThreads>(q_start, num_cached, num_seqs, table, max_blocks, p, sh, blockIdx.x,
                            gridDim.x);
}

}  // namespace

namespace hl {
hipError_t launch_plan(const int32_t* q_start, const int32_t* num_cached, int32_t num_seqs,
                       const int32_t* table, int32_t max_blocks, const Plan& plan,
                       hipStream_t st) {
  if (num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(hl::kPlanWorkgroups), dim3(kThreads), 0, st, q_start,
                     num_cached, num_seqs, table, max_blocks, plan);
  return hipGetLastError();
}
}  // namespace hl
