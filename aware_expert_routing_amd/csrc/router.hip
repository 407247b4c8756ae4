// Router linear projection: logits = x W_g + bias
// ("Router Caching and Optimization", section "Analyzing Router Inference
// Cost", step 1). W_g is [d, E], contiguous along E.
//
// bf16: one workgroup per 16-token x 16-expert tile of the logits, over the
// whole reduction, on MFMA (v_mfma_f32_16x16x32_bf16). The four waves take a
// quarter of the reduction each; A fragments (8 consecutive features of one
// token) load straight from x; W_g's 16 columns are staged in LDS in blocks
// of 128 rows (16-byte loads) and read back as B fragments (8 consecutive
// rows of one column). The waves' partial tiles are added in wave order, then
// the bias: the logits are the same bits on every run.
//
// float32 (small layers): a workgroup owns a 16-token x 16-expert tile of the logits and
// one slice of kRouterRows rows of the reduction: it stages its slice of x and
// of W_g in LDS (as float32, 16-byte loads where the rows allow), forms the
// 256 float32 dot products, and stores them as the slice's partial tile. It
// then counts itself on the tile's counter; the workgroup that completes the
// count adds the bias and the slices' partial tiles in slice order (so the
// logits are the same bits on every run), writes them and resets the counter.
// The reduction is split over many workgroups because the product is tiny and
// latency-bound: at d = 2048, E = 128, B = 16 it is 128 workgroups reading
// 8 KB each.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;  // tokens and experts per tile

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kBlockRows = 128;               // W_g rows per LDS block (4 k-steps)
constexpr int kGroupBlocks = 4;               // blocks whose loads are issued together

// grid = (ceil(E/16), ceil(B/16)); block = 256 (4 waves). VEC: the tile's 16
// columns are 16-byte aligned in every row (E % 8 == 0 and a whole tile).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ bias,
    int B, int d, int E, float *__restrict__ logits) {
  __shared__ uint16_t wl[4][kGroupBlocks][kBlockRows][kTile];  // per wave: W_g rows x 16 columns
  __shared__ float red[4][kTile][kTile];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * kTile, t0 = blockIdx.y * kTile;
  const int ne = min(kTile, E - e0);
  const int tok = min(t0 + j, B - 1);  // clamped: rows past B are computed and dropped
  // This wave's k-steps (32 reduction rows each).
  const int nks = (d + 31) / 32;
  const int per = (nks + 3) / 4;
  const int ks0 = wave * per, ks1 = min(nks, ks0 + per);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = ks0; kb < ks1; kb += 4 * kGroupBlocks) {
    // Issue every load of up to kGroupBlocks blocks, then use them.
    bf16x8_t a[4 * kGroupBlocks];
    uint4 wv[kGroupBlocks][4];
    bool wok[kGroupBlocks][4];
#pragma unroll
    for (int q = 0; q < 4 * kGroupBlocks; ++q) {
      const int k = (kb + q) * 32 + 8 * g;
      // Features past d (or of k-steps this wave does not use) read feature 0:
      // any finite value does, the W_g rows they meet are zero.
      const int kk = (kb + q < ks1 && k < d) ? k : 0;
      a[q] = *reinterpret_cast<const bf16x8_t *>(x + size_t(tok) * d + kk);
    }
#pragma unroll
    for (int b = 0; b < kGroupBlocks; ++b) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int piece = lane + 64 * q;  // 256 pieces of 16 B: row piece/2, half piece%2
        const int row = (kb + 4 * b) * 32 + piece / 2;
        const int c0 = (piece & 1) * 8;
        // Rows past d or outside this wave's range read row 0 (every load stays
        // in bounds and is issued unconditionally) and are stored as zero.
        const bool ok = kb + 4 * b < ks1 && row < d;
        wok[b][q] = ok;
        const size_t ro = size_t(ok ? row : 0) * E + e0 + c0;
        if (VEC) {
          wv[b][q] = *reinterpret_cast<const uint4 *>(w + ro);
        } else {
          uint32_t t[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t lo = (c0 + 2 * c < ne) ? w[ro + 2 * c] : 0u;
            const uint32_t hi = (c0 + 2 * c + 1 < ne) ? w[ro + 2 * c + 1] : 0u;
            t[c] = lo | (hi << 16);
          }
          wv[b][q] = make_uint4(t[0], t[1], t[2], t[3]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kGroupBlocks; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int piece = lane + 64 * q;
        *reinterpret_cast<uint4 *>(&wl[wave][b][piece / 2][(piece & 1) * 8]) =
            wok[b][q] ? wv[b][q] : make_uint4(0, 0, 0, 0);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 4 * kGroupBlocks; ++q) {
      if (kb + q < ks1) {
        bf16x8_t bfrag;
#pragma unroll
        for (int r = 0; r < 8; ++r) bfrag[r] = short(wl[wave][q / 4][(q % 4) * 32 + 8 * g + r][j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], bfrag, acc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // acc holds rows 4g + i (tokens), column j (expert) of this wave's partial tile.
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * g + i][j] = acc[i];
  __syncthreads();
  const int ti = threadIdx.x / kTile, ej = threadIdx.x % kTile;
  if (t0 + ti < B && ej < ne) {
    float v = bias ? bias[e0 + ej] : 0.0f;
    v += red[0][ti][ej] + red[1][ti][ej] + red[2][ti][ej] + red[3][ti][ej];
    logits[size_t(t0 + ti) * E + e0 + ej] = v;
  }
}

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
    const dim3 grid(ceil_div(E, kTile), ceil_div(B, kTile));
    const uint16_t *xb = static_cast<const uint16_t *>(x), *wb = static_cast<const uint16_t *>(w_g);
    if (E % kTile == 0)
      router_mfma_kernel<true><<<grid, kThreads, 0, s>>>(xb, wb, bias, B, d, E, logits);
    else
      router_mfma_kernel<false><<<grid, kThreads, 0, s>>>(xb, wb, bias, B, d, E, logits);
    return hipGetLastError();
  }
  dim3 grid(ceil_div(E, kTile), ceil_div(d, kRouterRows), ceil_div(B, kTile));
  router_kernel<float><<<grid, kThreads, 0, s>>>(static_cast<const float *>(x),
                                                   static_cast<const float *>(w_g), bias, B, d, E,
                                                   part, cnt, logits);
  return hipGetLastError();
}

}  // namespace moe
