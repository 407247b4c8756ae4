// Router linear projection: logits = x W_g + bias
// ("Router Caching and Optimization", section "Analyzing Router Inference
// Cost", step 1). W_g is [d, E], contiguous along E.
//
// The product is split over d into slices of kRouterRows rows so that many
// workgroups share the (small, latency-bound) read of W_g. A workgroup stages
// its slice of W_g (16-byte loads, all issued before any is used) and of x in
// LDS, then each thread forms float32 dot products over the slice's rows.
// Each slice writes partial sums part[slice][t][e]; a second kernel adds them
// and the bias in a fixed order, so the logits are bit-reproducible from run
// to run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = 64;

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}

// grid = (slices, ceil(B / kTokPerBlock)); block = kThreads.
template <typename T>
__global__ __launch_bounds__(kThreads) void router_partial_kernel(
    const T *__restrict__ x, const T *__restrict__ w, int B, int d, int E,
    float *__restrict__ part) {
  __shared__ float ws[kRouterRows][kMaxE];
  __shared__ float xs[kTokPerBlock][kRouterRows + 1];
  const int s = blockIdx.x;
  const int t0 = blockIdx.y * kTokPerBlock;
  const int nt = min(kTokPerBlock, B - t0);
  const int r0 = s * kRouterRows;
  const int nr = min(kRouterRows, d - r0);

  // W_g slice: nr rows of E elements, moved in 16-byte chunks when a row is a
  // whole number of chunks, element by element otherwise.
  constexpr int per = 16 / sizeof(T);
  if ((E % per) == 0) {
    const int cpr = E / per;  // chunks per row
    const int nchunks = nr * cpr;
    constexpr int kMaxIter = kRouterRows * kMaxE / per / kThreads;
    uint4 v[kMaxIter];
#pragma unroll
    for (int i = 0; i < kMaxIter; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (c < nchunks) v[i] = *reinterpret_cast<const uint4 *>(w + size_t(r0) * E + size_t(c) * per);
    }
#pragma unroll
    for (int i = 0; i < kMaxIter; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (c < nchunks) {
        const int r = c / cpr, e0 = (c - r * cpr) * per;
        const T *pv = reinterpret_cast<const T *>(&v[i]);
#pragma unroll
        for (int j = 0; j < per; ++j) ws[r][e0 + j] = to_f32<T>(pv[j]);
      }
    }
  } else {
    for (int i = threadIdx.x; i < nr * E; i += kThreads)
      ws[i / E][i % E] = to_f32<T>(w[size_t(r0) * E + i]);
  }
  for (int i = threadIdx.x; i < nt * kRouterRows; i += kThreads) {
    const int t = i / kRouterRows, r = i % kRouterRows;
    xs[t][r] = (r < nr) ? to_f32<T>(x[size_t(t0 + t) * d + r0 + r]) : 0.0f;
  }
  __syncthreads();

  for (int o = threadIdx.x; o < nt * E; o += kThreads) {
    const int t = o / E, e = o - t * E;
    float acc = 0.0f;
    for (int r = 0; r < nr; ++r) acc = fmaf(xs[t][r], ws[r][e], acc);
    part[(size_t(s) * B + (t0 + t)) * E + e] = acc;
  }
}

// logits = bias + sum over slices of the partial sums, in a fixed order:
// thread (o, g) of a workgroup adds slices g, g+8, g+16, ... of output o
// (all its loads are independent), then group sums are added in g order.
constexpr int kRedOut = 32;                      // outputs per workgroup
constexpr int kRedGroups = kThreads / kRedOut;   // slice groups

__global__ __launch_bounds__(kThreads) void router_reduce_kernel(
    const float *__restrict__ part, const float *__restrict__ bias, int slices, int B, int E,
    float *__restrict__ logits) {
  __shared__ float red[kRedGroups][kRedOut];
  const int ol = threadIdx.x % kRedOut, g = threadIdx.x / kRedOut;
  const int o = blockIdx.x * kRedOut + ol;
  const size_t n = size_t(B) * E;
  float acc = 0.0f;
  if (o < int(n)) {
#pragma unroll 8
    for (int s = g; s < slices; s += kRedGroups) acc += part[size_t(s) * n + o];
  }
  red[g][ol] = acc;
  __syncthreads();
  if (g == 0 && o < int(n)) {
    float v = bias ? bias[o % E] : 0.0f;
#pragma unroll
    for (int j = 0; j < kRedGroups; ++j) v += red[j][ol];
    logits[o] = v;
  }
}

}  // namespace

hipError_t launch_router(const void *x, const void *w_g, moe_dtype_t dt, int B, int d, int E,
                         float *part, int slices, hipStream_t s) {
  dim3 grid(slices, ceil_div(B, kTokPerBlock));
  if (dt == MOE_BF16)
    router_partial_kernel<uint16_t><<<grid, kThreads, 0, s>>>(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_g), B, d, E, part);
  else
    router_partial_kernel<float><<<grid, kThreads, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(w_g), B, d, E, part);
  return hipGetLastError();
}

hipError_t launch_router_reduce(const float *part, const float *bias, int slices, int B, int E,
                                float *logits, hipStream_t s) {
  router_reduce_kernel<<<ceil_div(B * E, kRedOut), kThreads, 0, s>>>(part, bias, slices, B, E,
                                                                     logits);
  return hipGetLastError();
}

}  // namespace moe
