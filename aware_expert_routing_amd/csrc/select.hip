// Standalone selection kernel (moe_select): one workgroup runs select_block
// on the caller's logits.
#include "select_impl.h"

namespace moe {
namespace {

template <int NV, int TPW>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float *__restrict__ logits, int B, int E, int kind, int k, int k0, int m, int g, float bin_w,
    int32_t *__restrict__ topk_ids, float *__restrict__ topk_w, int32_t *__restrict__ n_active,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ pair_token, int32_t *__restrict__ pair_slot,
    float *__restrict__ batch_mass) {
  select_block<NV, TPW>(StoredLogits{logits, E}, B, E, kind, k, k0, m, g, bin_w, topk_ids, topk_w, n_active, active_experts,
                   expert_offsets, pair_token, pair_slot, batch_mass);
}

}  // namespace

hipError_t launch_select(const float *logits, int B, int E, moe_policy_t p,
                         const moe_routing_t &r, hipStream_t s) {
  float *mass = (p.kind == MOE_POLICY_BUDGET || p.kind == MOE_POLICY_HIER) ? r.batch_mass : nullptr;
  dispatch_select_shape(B, E, [&](auto nv, auto tpw) {
    select_kernel<decltype(nv)::value, decltype(tpw)::value><<<1, kThreads, 0, s>>>(
        logits, B, E, p.kind, p.k, p.k0, p.m, p.g, lynx_bin_width(E, p.k), r.topk_ids, r.topk_w, r.n_active,
        r.active_experts, r.expert_offsets, r.pair_token, r.pair_slot, mass);
  });
  return hipGetLastError();
}

}  // namespace moe
