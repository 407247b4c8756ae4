// Router linear projection: logits = x W_g + bias
// ("Router Caching and Optimization", section "Analyzing Router Inference
// Cost", step 1). W_g is [d, E], contiguous along E.
//
// bf16: one 1024-thread workgroup per 16-token x 16-expert tile of the
// logits and slice of 512 rows of the reduction, on MFMA (router_partial in
// router_impl.h); it stores the slice's partial tile, and the workgroup that
// completes the tile's count adds the bias and the slices in order.
//
// float32 (small layers): a workgroup owns a 16-token x 16-expert tile of
// the logits and one slice of kRouterRows rows of the reduction: it stages
// its slice of x and of W_g in LDS (16-byte loads where the rows allow),
// forms the 256 float32 dot products, and stores them as the slice's partial
// tile. It then counts itself on the tile's counter; the workgroup that
// completes the count adds the bias and the slices' partial tiles in slice
// order (so the logits are the same bits on every run), writes them and
// resets the counter.
#include "router_impl.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;  // tokens and experts per tile

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}

// `rows` x `cols` elements at src (row stride ld) into dst[r][c] (row stride
// dld, float32); elements outside nr x nc read as zero. Rows are moved in
// 16-byte chunks when every chunk is aligned and whole.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ void stage(const T *__restrict__ src, size_t ld, int nr, int nc,
                                      float *dst, int dld) {
  constexpr int per = 16 / sizeof(T);
  constexpr int cpr = COLS / per;  // chunks per row
  if ((ld % per) == 0 && nc == COLS) {
    for (int c = threadIdx.x; c < ROWS * cpr; c += kThreads) {
      const int r = c / cpr, c0 = (c - r * cpr) * per;
      T v[per];
      if (r < nr) {
        *reinterpret_cast<uint4 *>(v) = *reinterpret_cast<const uint4 *>(src + size_t(r) * ld + c0);
      } else {
#pragma unroll
        for (int q = 0; q < per; ++q) v[q] = T(0);
      }
#pragma unroll
      for (int q = 0; q < per; ++q) dst[r * dld + c0 + q] = to_f32<T>(v[q]);
    }
  } else {
    for (int i = threadIdx.x; i < ROWS * COLS; i += kThreads) {
      const int r = i / COLS, c = i - r * COLS;
      dst[r * dld + c] = (r < nr && c < nc) ? to_f32<T>(src[size_t(r) * ld + c]) : 0.0f;
    }
  }
}

// bf16: grid = (ceil(E/16), ceil(B/16), slices); block = 1024.
template <bool VEC>
__global__ __launch_bounds__(kRtThreads) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ bias,
    int B, int d, int E, float *__restrict__ part, uint32_t *__restrict__ cnt,
    float *__restrict__ logits) {
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
    const uint32_t before =
        __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == uint32_t(slices - 1);
    if (s_last) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last || threadIdx.x >= kRtTile * kRtTile) return;
  const int t = blockIdx.y * kRtTile + threadIdx.x / kRtTile;
  const int e = blockIdx.x * kRtTile + threadIdx.x % kRtTile;
  if (t < B && e < E) logits[size_t(t) * E + e] = router_logit(part, bias, t, e, gridDim.x, slices);
}

// float32: grid = (ceil(E/16), slices, ceil(B/16)); block = 256 = 16 x 16
// outputs.
template <typename T>
__global__ __launch_bounds__(kThreads) void router_kernel(
    const T *__restrict__ x, const T *__restrict__ w, const float *__restrict__ bias, int B, int d,
    int E, float *__restrict__ part, uint32_t *__restrict__ cnt, float *__restrict__ logits) {
  __shared__ float xs[kTile][kRouterRows + 1];  // +1: the 4 token rows a wave reads sit in distinct banks
  __shared__ float ws[kRouterRows][kTile];
  __shared__ int s_last;
  const int te = blockIdx.x, ks = blockIdx.y, tt = blockIdx.z;
  const int slices = gridDim.y;
  const int e0 = te * kTile, t0 = tt * kTile, k0 = ks * kRouterRows;
  const int ne = min(kTile, E - e0), nt = min(kTile, B - t0), nk = min(kRouterRows, d - k0);

  stage<T, kTile, kRouterRows>(x + size_t(t0) * d + k0, size_t(d), nt, nk, &xs[0][0], kRouterRows + 1);
  stage<T, kRouterRows, kTile>(w + size_t(k0) * E + e0, size_t(E), nk, ne, &ws[0][0], kTile);
  __syncthreads();

  const int i = threadIdx.x / kTile, j = threadIdx.x % kTile;
  float acc = 0.0f;
#pragma unroll 8
  for (int k = 0; k < kRouterRows; ++k) acc = fmaf(xs[i][k], ws[k][j], acc);

  const int tile = te * gridDim.z + tt;
  float *tp = part + size_t(tile) * slices * (kTile * kTile);
  // Device-scope store: the workgroup that completes the tile reads it.
  __hip_atomic_store(tp + ks * (kTile * kTile) + threadIdx.x, acc, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == uint32_t(slices - 1);
  }
  __syncthreads();
  if (!s_last) return;

  float v = (bias && j < ne) ? bias[e0 + j] : 0.0f;
  for (int s = 0; s < slices; ++s)
    v += __hip_atomic_load(tp + s * (kTile * kTile) + threadIdx.x, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  if (i < nt && j < ne) logits[size_t(t0 + i) * E + e0 + j] = v;
  if (threadIdx.x == 0) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_router(const void *x, const void *w_g, const float *bias, moe_dtype_t dt, int B,
                         int d, int E, float *part, uint32_t *cnt, float *logits, hipStream_t s) {
  if (dt == MOE_BF16) {
    const dim3 grid(ceil_div(E, kTile), ceil_div(B, kTile), router_slices(d));
    const uint16_t *xb = static_cast<const uint16_t *>(x), *wb = static_cast<const uint16_t *>(w_g);
    if (E % kTile == 0)
      router_mfma_kernel<true><<<grid, kRtThreads, 0, s>>>(xb, wb, bias, B, d, E, part, cnt, logits);
    else
      router_mfma_kernel<false><<<grid, kRtThreads, 0, s>>>(xb, wb, bias, B, d, E, part, cnt, logits);
    return hipGetLastError();
  }
  dim3 grid(ceil_div(E, kTile), ceil_div(d, kRouterRows), ceil_div(B, kTile));
  router_kernel<float><<<grid, kThreads, 0, s>>>(static_cast<const float *>(x),
                                                   static_cast<const float *>(w_g), bias, B, d, E,
                                                   part, cnt, logits);
  return hipGetLastError();
}

}  // namespace moe
