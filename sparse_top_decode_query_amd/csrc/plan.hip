// Per-query read plan by reverse water-filling (Fathom summary,
// water-filling paragraph): one wavefront per KV head; the computation is
// plan_head in plan_dev.hpp.
#include "plan_dev.hpp"

namespace sdq {

template <bool UNIFORM>
__global__ __launch_bounds__(64) void fathom_plan_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ var, int Hgrp,
                                                         int budget, uint8_t* __restrict__ depth,
                                                         float* __restrict__ qbar) {
  __shared__ __attribute__((aligned(16))) uint32_t s_scratch[3 * kHeadDim];
  const int g = blockIdx.x;
  const int l = threadIdx.x;
  const HeadPlan p = plan_head<UNIFORM>(q, var, g, Hgrp, budget, s_scratch);
  qbar[size_t(g) * kHeadDim + l] = p.a0;
  qbar[size_t(g) * kHeadDim + l + 64] = p.a1;
  depth[size_t(g) * kHeadDim + l] = uint8_t(p.d0);
  depth[size_t(g) * kHeadDim + l + 64] = uint8_t(p.d1);
}

}  // namespace sdq

using namespace sdq;

static int plan_common(const float* q, const float* key_var, int G, int H_grp, int d, int budget,
                       uint8_t* depth, float* qbar, hipStream_t stream, bool uniform) {
  const char* nm = uniform ? "fathom_plan_uniform" : "fathom_plan";
  SDQ_REQUIRE(q && key_var && depth && qbar, "%s: null pointer", nm);
  SDQ_REQUIRE(G >= 1 && H_grp >= 1, "%s: G=%d, H_grp=%d must be >= 1", nm, G, H_grp);
  SDQ_REQUIRE(d == kHeadDim, "%s: d=%d unsupported (only 128)", nm, d);
  SDQ_REQUIRE(budget >= 0, "%s: budget/channel count %d must be >= 0", nm, budget);
  SDQ_REQUIRE(!uniform || budget <= d, "%s: n_channels=%d exceeds d=%d", nm, budget, d);
  if (uniform)
    hipLaunchKernelGGL(fathom_plan_kernel<true>, dim3(G), dim3(64), 0, stream, q, key_var, H_grp,
                       budget, depth, qbar);
  else
    hipLaunchKernelGGL(fathom_plan_kernel<false>, dim3(G), dim3(64), 0, stream, q, key_var, H_grp,
                       budget, depth, qbar);
  return check_launch(nm);
}

extern "C" int fathom_plan(const float* q, const float* key_var, int G, int H_grp, int d,
                           int budget_bits, uint8_t* depth, float* qbar, hipStream_t stream) {
  return plan_common(q, key_var, G, H_grp, d, budget_bits, depth, qbar, stream, false);
}

extern "C" int fathom_plan_uniform(const float* q, const float* key_var, int G, int H_grp, int d,
                                   int n_channels, uint8_t* depth, float* qbar,
                                   hipStream_t stream) {
  return plan_common(q, key_var, G, H_grp, d, n_channels, depth, qbar, stream, true);
}
