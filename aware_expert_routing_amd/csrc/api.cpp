// extern "C" entry points of libmoe_decode: argument checks (before any HIP
// call), workspace planning and kernel launches on the caller's stream.
#include <stdint.h>
#include <string.h>

#include "moe_internal.h"

namespace {

using namespace moe;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dtype(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// Sizes: k <= E is a contract (INVALID_ARG); the rest is the envelope.
moe_status_t check_sizes(int B, int d, int E, int I, int k) {
  if (B < 1 || d < 1 || E < 1 || I < 1 || k < 1) return MOE_ERR_INVALID_ARG;
  if (k > E) return MOE_ERR_INVALID_ARG;
  if (B > kMaxB || E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (d < 8 || I < 8 || d > kMaxDim || I > kMaxDim || d % 8 || I % 8) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_policy(const moe_policy_t &p, int E) {
  if (p.k < 1 || p.k > E) return MOE_ERR_INVALID_ARG;
  if (p.k > kMaxK) return MOE_ERR_UNSUPPORTED;
  switch (p.kind) {
    case MOE_POLICY_TOPK:
      return MOE_OK;
    case MOE_POLICY_OEA:
      return (p.k0 >= 1 && p.k0 <= p.k) ? MOE_OK : MOE_ERR_INVALID_ARG;
    case MOE_POLICY_BUDGET:
    case MOE_POLICY_GREEDY:
      return (p.m >= 1 && p.m <= E) ? MOE_OK : MOE_ERR_INVALID_ARG;
    case MOE_POLICY_HIER:
      return (p.m >= 1 && p.m <= E && p.k0 >= 1 && p.k0 <= p.m && p.g >= 1) ? MOE_OK
                                                                             : MOE_ERR_INVALID_ARG;
    case MOE_POLICY_LYNX:
      return (p.m >= p.k && p.m <= E) ? MOE_OK : MOE_ERR_INVALID_ARG;
    default:
      return MOE_ERR_INVALID_ARG;
  }
}

moe_status_t check_routing(const moe_routing_t *r, bool need_mass) {
  if (!r) return MOE_ERR_INVALID_ARG;
  const void *ptrs[] = {r->topk_ids, r->topk_w, r->n_active, r->active_experts,
                        r->expert_offsets, r->pair_token, r->pair_slot};
  for (const void *p : ptrs)
    if (!p || !aligned(p, 4)) return MOE_ERR_INVALID_ARG;
  if (need_mass && !r->batch_mass) return MOE_ERR_INVALID_ARG;
  if (r->batch_mass && !aligned(r->batch_mass, 4)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_dense(const void *p) {
  return (p && aligned(p, 16)) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

moe_status_t check_workspace(const void *ws, size_t have, size_t need) {
  if (!ws || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  return have >= need ? MOE_OK : MOE_ERR_WORKSPACE;
}

// moe_route writes its partial sums where the full plan puts them, after the
// expert FFN's synchronisation words, so that a workspace can serve every
// entry point.
size_t route_bytes(int B, int d, int E) {
  const size_t tiles = size_t(ceil_div(E, kRouterTile)) * ceil_div(B, kRouterTile);
  return kCounterBytes +
         align256(tiles * ceil_div(d, kRouterRows) * kRouterTile * kRouterTile * sizeof(float));
}

#define MOE_TRY(expr)                     \
  do {                                    \
    const moe_status_t st_ = (expr);      \
    if (st_ != MOE_OK) return st_;        \
  } while (0)

moe_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  return e == hipErrorCooperativeLaunchTooLarge ? MOE_ERR_RESIDENCY : MOE_ERR_HIP;
}

// Checks of every moe_layer_decode argument except the workspace.
moe_status_t check_layer_args(const void *x, const void *w_g, const float *bias, const void *w_gate,
                              const void *w_up, const void *w_down, moe_dtype_t dt, int B, int d,
                              int E, int I, const moe_policy_t &policy, const float *logits,
                              const moe_routing_t *routing, const void *y) {
  if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_sizes(B, d, E, I, policy.k < 1 ? 1 : policy.k));
  MOE_TRY(check_policy(policy, E));
  MOE_TRY(check_dense(x));
  MOE_TRY(check_dense(w_g));
  MOE_TRY(check_dense(w_gate));
  MOE_TRY(check_dense(w_up));
  MOE_TRY(check_dense(w_down));
  MOE_TRY(check_dense(y));
  if (!logits || !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 4)) return MOE_ERR_INVALID_ARG;
  return check_routing(routing, policy.kind == MOE_POLICY_BUDGET || policy.kind == MOE_POLICY_HIER);
}

// The layer's launches on stream s with workspace ws (planned by plan).
moe_status_t layer_launches(const void *x, const void *w_g, const float *bias, const void *w_gate,
                            const void *w_up, const void *w_down, moe_dtype_t dt, int B, int d,
                            int E, int I, const moe_policy_t &policy, float *logits,
                            const moe_routing_t *routing, void *y, char *ws, const Workspace &plan,
                            hipStream_t s) {
  if (dt == MOE_BF16) {
    float *part = reinterpret_cast<float *>(ws + plan.router_part);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + kRouteSelectCntOffset);
    MOE_TRY(hip_status(launch_route_select(x, w_g, bias, B, d, E, logits, part, cnt, policy, *routing, s)));
  } else {
    float *part = reinterpret_cast<float *>(ws + plan.router_part);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + kRouterCntOffset);
    MOE_TRY(hip_status(launch_router(x, w_g, bias, dt, B, d, E, part, cnt, logits, s)));
    MOE_TRY(hip_status(launch_select(logits, B, E, policy, *routing, s)));
  }
  return hip_status(launch_expert_ffn(x, w_gate, w_up, w_down, dt, B, d, E, I, policy.k, *routing,
                                      y, ws, plan, s));
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(int B, int d, int E, int I, int k, moe_dtype_t dt) {
  if (!valid_dtype(dt) || check_sizes(B, d, E, I, k) != MOE_OK) return 0;
  return plan_workspace(B, d, E, I, k, dt).total;
}

moe_status_t moe_route(const void *x, const void *w_g, const float *bias, moe_dtype_t dt, int B,
                       int d, int E, float *logits, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_sizes(B, d, E, 8, 1));
  MOE_TRY(check_dense(x));
  MOE_TRY(check_dense(w_g));
  if (!logits || !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 4)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_workspace(workspace, workspace_bytes, route_bytes(B, d, E)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  float *part = reinterpret_cast<float *>(ws + kCounterBytes);
  uint32_t *cnt = reinterpret_cast<uint32_t *>(ws + kRouterCntOffset);
  return hip_status(launch_router(x, w_g, bias, dt, B, d, E, part, cnt, logits, s));
}

moe_status_t moe_select(const float *logits, int B, int E, moe_policy_t policy,
                        const moe_routing_t *out, void *stream) {
  if (!logits || !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
  if (B < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (B > kMaxB || E > kMaxE) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(check_policy(policy, E));
  MOE_TRY(check_routing(out, policy.kind == MOE_POLICY_BUDGET || policy.kind == MOE_POLICY_HIER));
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_select(logits, B, E, policy, *out, s));
}

moe_status_t moe_expert_ffn(const void *x, const void *w_gate, const void *w_up,
                            const void *w_down, moe_dtype_t dt, int B, int d, int E, int I,
                            int k, const moe_routing_t *routing, void *y, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_sizes(B, d, E, I, k));
  MOE_TRY(check_dense(x));
  MOE_TRY(check_dense(w_gate));
  MOE_TRY(check_dense(w_up));
  MOE_TRY(check_dense(w_down));
  MOE_TRY(check_dense(y));
  MOE_TRY(check_routing(routing, false));
  const Workspace plan = plan_workspace(B, d, E, I, k, dt);
  MOE_TRY(check_workspace(workspace, workspace_bytes, plan.total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_expert_ffn(x, w_gate, w_up, w_down, dt, B, d, E, I, k, *routing, y,
                                      static_cast<char *>(workspace), plan, s));
}

moe_status_t moe_layer_decode(const void *x, const void *w_g, const float *bias,
                              const void *w_gate, const void *w_up, const void *w_down,
                              moe_dtype_t dt, int B, int d, int E, int I, moe_policy_t policy,
                              float *logits, const moe_routing_t *routing, void *y,
                              void *workspace, size_t workspace_bytes, void *stream) {
  MOE_TRY(check_layer_args(x, w_g, bias, w_gate, w_up, w_down, dt, B, d, E, I, policy, logits, routing, y));
  const Workspace plan = plan_workspace(B, d, E, I, policy.k, dt);
  MOE_TRY(check_workspace(workspace, workspace_bytes, plan.total));
  MOE_TRY(hip_status(expert_ffn_launchable(dt, B, d, E, I, policy.k, plan)));
  return layer_launches(x, w_g, bias, w_gate, w_up, w_down, dt, B, d, E, I, policy, logits, routing, y,
                        static_cast<char *>(workspace), plan, static_cast<hipStream_t>(stream));
}

moe_status_t moe_layer_decode_static(const void *x, const void *w_g, const float *bias,
                                     const void *w_gate, const void *w_up, const void *w_down,
                                     moe_dtype_t dt, int B, int d, int E, int I, moe_policy_t policy,
                                     float *logits, const moe_routing_t *routing, void *y,
                                     void *stream) {
  MOE_TRY(check_layer_args(x, w_g, bias, w_gate, w_up, w_down, dt, B, d, E, I, policy, logits, routing, y));
  const Workspace plan = plan_workspace(B, d, E, I, policy.k, dt);
  if (plan.total > kStaticScratchBytes) return MOE_ERR_SCRATCH;
  MOE_TRY(hip_status(expert_ffn_launchable(dt, B, d, E, I, policy.k, plan)));
  char *ws = nullptr;
  MOE_TRY(hip_status(static_scratch_address(&ws)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The previous call's counters are back at zero unless it was cut short;
  // zero them anyway, so that every call starts from a known state.
  MOE_TRY(hip_status(clear_scratch_counters(ws, s)));
  return layer_launches(x, w_g, bias, w_gate, w_up, w_down, dt, B, d, E, I, policy, logits, routing, y,
                        ws, plan, s);
}

moe_status_t moe_workspace_check(const void *status_host, size_t bytes) {
  if (!status_host || bytes < MOE_WS_STATUS_BYTES) return MOE_ERR_INVALID_ARG;
  uint32_t word;
  memcpy(&word, static_cast<const char *>(status_host) + kSyncErrOffset, sizeof(word));
  return word != 0 ? MOE_ERR_SYNC_TIMEOUT : MOE_OK;
}

moe_status_t moe_read_stream(const void *src, size_t bytes, uint32_t *out, void *stream) {
  if (!src || !aligned(src, 16) || !out || !aligned(out, 4) || bytes == 0 || bytes % 16)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_read_stream(src, bytes, out, static_cast<hipStream_t>(stream)));
}

const char *moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK:
      return "MOE_OK: success";
    case MOE_ERR_INVALID_ARG:
      return "MOE_ERR_INVALID_ARG: null or misaligned pointer, or an argument out of its range";
    case MOE_ERR_UNSUPPORTED:
      return "MOE_ERR_UNSUPPORTED: sizes outside the supported envelope";
    case MOE_ERR_WORKSPACE:
      return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP:
      return "MOE_ERR_HIP: a kernel launch failed";
    case MOE_ERR_RESIDENCY:
      return "MOE_ERR_RESIDENCY: the expert FFN's workgroups cannot all be resident on this device";
    case MOE_ERR_SCRATCH:
      return "MOE_ERR_SCRATCH: the sizes need more scratch than the static array of "
             "moe_layer_decode_static holds (MOE_STATIC_SCRATCH_BYTES)";
    case MOE_ERR_SYNC_TIMEOUT:
      return "MOE_ERR_SYNC_TIMEOUT: a grid-wide wait of the expert FFN gave up; outputs of the calls "
             "since the workspace was zero-filled are unspecified";
    default:
      return "unknown moe_status_t";
  }
}

}  // extern "C"
