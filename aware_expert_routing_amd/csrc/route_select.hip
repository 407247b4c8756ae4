// Router and selection in one launch (bf16 layers, moe_layer_decode).
// Grid (ceil(E/16), ceil(B/16), slices of 512 rows of d): each 1024-thread
// workgroup computes the partial 16 x 16 logit tile of one slice
// (router_partial), stores it with device-scope stores and counts itself on
// a counter in the workspace. The workgroup that completes the count forms
// every logit as bias + slice 0 + slice 1 + ... (router_logit, the same sum
// in the same order as moe_route's), straight into the selection's registers,
// writes the logits output, runs the whole selection (select_block) and
// resets the counter. The logits are bit-identical to moe_route's, and the
// routing to moe_select's on them.
#include "router_impl.h"
#include "select_impl.h"

namespace moe {
namespace {

static_assert(kRtThreads == kThreads, "router tile and selection share the workgroup size");

// Logits completed from the slices' partial tiles; each value read is also
// written to the logits output.
struct SliceLogits {
  const float *part;
  const float *bias;
  float *out;
  int E, tiles_e, slices;
  __device__ __forceinline__ float operator()(int t, int e) const {
    return router_logit(part, bias, t, e, tiles_e, slices);
  }
  // The same sums as router_logit (bias, then slice 0, 1, ... in order) for
  // every slot: the partial-tile loads of G slots x NV experts x 4 slices are
  // all issued (indices clamped, no branch between them) before the first
  // add, one round trip per 4 slices instead of one per logit.
  template <int TPW, int NV>
  __device__ __forceinline__ void gather(float (&L)[TPW][NV], int B, int wave, int lane) const {
    constexpr int G = TPW < 8 / NV ? TPW : 8 / NV;  // slots per round trip
    constexpr int S = 4;                            // slices per round trip
    constexpr int kTile = kRtTile * kRtTile;
#pragma unroll
    for (int g0 = 0; g0 < TPW; g0 += G) {
      if (g0 * kWaves >= B) break;  // block-uniform
      float acc[G][NV];
      const float *tp[G][NV];
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int t = min(wave + kWaves * (g0 + i), B - 1), e = min(lane + 64 * v, E - 1);
          const int tile = e / kRtTile + tiles_e * (t / kRtTile);
          tp[i][v] = part + size_t(tile) * slices * kTile + (t % kRtTile) * kRtTile + (e % kRtTile);
          acc[i][v] = bias ? bias[e] : 0.0f;
        }
      for (int s0 = 0; s0 < slices; s0 += S) {
        float p[G][NV][S];
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int q = 0; q < S; ++q)
              p[i][v][q] = __hip_atomic_load(const_cast<float *>(tp[i][v]) + min(s0 + q, slices - 1) * kTile,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int q = 0; q < S; ++q)
              if (s0 + q < slices) acc[i][v] += p[i][v][q];
      }
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int v = 0; v < NV; ++v) L[g0 + i][v] = acc[i][v];
    }
  }
  __device__ __forceinline__ void emit(int t, int e, float v) const { out[size_t(t) * E + e] = v; }
};

template <bool VEC, int NV, int TPW>
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ bias,
    int B, int d, int E, float *__restrict__ logits, float *__restrict__ part,
    uint32_t *__restrict__ cnt, int kind, int k, int k0, int m, int g, float bin_w,
    int32_t *__restrict__ topk_ids, float *__restrict__ topk_w, int32_t *__restrict__ n_active,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ pair_token, int32_t *__restrict__ pair_slot,
    float *__restrict__ batch_mass) {
  __shared__ RouterLds sm;
  __shared__ int s_last;
  const int slices = gridDim.z;
  const int tile = blockIdx.x + gridDim.x * blockIdx.y;
  const float v = router_partial<VEC>(x, w, B, d, E, blockIdx.z, sm);
  if (threadIdx.x < kRtTile * kRtTile)
    __hip_atomic_store(part + (size_t(tile) * slices + blockIdx.z) * (kRtTile * kRtTile) + threadIdx.x, v,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this slice's partial tile is stored
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t total = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t before =
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == total - 1;
    if (s_last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  select_block<NV, TPW>(SliceLogits{part, bias, logits, E, int(gridDim.x), slices}, B, E, kind, k, k0,
                        m, g, bin_w, topk_ids, topk_w, n_active, active_experts, expert_offsets, pair_token,
                        pair_slot, batch_mass);
}

template <bool VEC>
void launch_rs(dim3 grid, const uint16_t *x, const uint16_t *w, const float *bias, int B, int d,
               int E, float *logits, float *part, uint32_t *cnt, const moe_policy_t &p,
               const moe_routing_t &r, hipStream_t s) {
  float *mass = (p.kind == MOE_POLICY_BUDGET || p.kind == MOE_POLICY_HIER) ? r.batch_mass : nullptr;
  dispatch_select_shape(B, E, [&](auto nv, auto tpw) {
    route_select_kernel<VEC, decltype(nv)::value, decltype(tpw)::value><<<grid, kThreads, 0, s>>>(
        x, w, bias, B, d, E, logits, part, cnt, p.kind, p.k, p.k0, p.m, p.g, lynx_bin_width(E, p.k),
        r.topk_ids, r.topk_w,
        r.n_active, r.active_experts, r.expert_offsets, r.pair_token, r.pair_slot, mass);
  });
}

}  // namespace

hipError_t launch_route_select(const void *x, const void *w_g, const float *bias, int B, int d,
                               int E, float *logits, float *part, uint32_t *cnt, moe_policy_t p,
                               const moe_routing_t &r, hipStream_t s) {
  const dim3 grid(ceil_div(E, kRtTile), ceil_div(B, kRtTile), router_slices(d));
  const uint16_t *xb = static_cast<const uint16_t *>(x), *wb = static_cast<const uint16_t *>(w_g);
  if (E % kRtTile == 0)
    launch_rs<true>(grid, xb, wb, bias, B, d, E, logits, part, cnt, p, r, s);
  else
    launch_rs<false>(grid, xb, wb, bias, B, d, E, logits, part, cnt, p, r, s);
  return hipGetLastError();
}

}  // namespace moe
