// bf16 router slice ("Router Caching and Optimization", section "Analyzing
// Router Inference Cost", step 1: logits = x W_g + bias), as a device
// function run by one workgroup of 1024 threads (16 waves): the partial
// 16-token x 16-expert logit tile of one slice of kRtSliceRows rows of the
// reduction, on MFMA (v_mfma_f32_16x16x32_bf16). Wave w takes k-step w (32
// rows) of the slice: its A fragments (8 consecutive features of one token)
// load straight from x; the slice's 32 rows of W_g's 16 columns (1 KB) are
// staged in LDS and read back as B fragments (8 consecutive rows of one
// column). The waves' partial tiles are added in wave order.
//
// A workgroup moves 32 KB (16 KB of x, 16 KB of W_g): a compute unit keeps
// about that much in flight, so the loads cost one round trip. The tile is
// completed from its slices' partial tiles by the caller, always as
// bias + slice 0 + slice 1 + ... in that order, so every kernel that uses
// this function produces the same bits.
#pragma once
#include "moe_internal.h"

namespace moe {
namespace {

typedef short rt_bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float rt_f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kRtThreads = 1024;
constexpr int kRtWaves = kRtThreads / 64;
constexpr int kRtTile = 16;                       // tokens and experts per tile
constexpr int kRtSliceRows = kRtWaves * 32;       // reduction rows per workgroup (one k-step per wave)

inline int router_slices(int d) { return ceil_div(d, kRtSliceRows); }

struct RouterLds {
  uint16_t wl[kRtWaves][32][kRtTile];     // per wave: its 32 rows of W_g x 16 columns
  float red[kRtWaves][kRtTile][kRtTile];  // per wave: partial tile
};

// Partial tile of slice `slice` of tile (blockIdx.x: experts, blockIdx.y:
// tokens). Returns, for thread i < 256, element (token i / 16, expert i % 16)
// of the slice's partial tile (0 for the other threads). VEC: the tile's 16
// columns are 16-byte aligned in every row (E % 16 == 0). Rows past d and
// tokens past B contribute zeros (their loads are clamped in bounds).
template <bool VEC>
__device__ __forceinline__ float router_partial(const uint16_t *__restrict__ x,
                                                const uint16_t *__restrict__ w, int B, int d, int E,
                                                int slice, RouterLds &sm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * kRtTile, t0 = blockIdx.y * kRtTile;
  const int ne = min(kRtTile, E - e0);
  const int tok = min(t0 + j, B - 1);
  const int ks = slice * kRtWaves + wave;  // this wave's k-step
  rt_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (ks * 32 < d) {  // wave-uniform
    // A fragment: features ks*32 + 8g .. +7 of token tok (past d: feature 0,
    // any finite value, met by zero rows of W_g).
    const int kk = ks * 32 + 8 * g < d ? ks * 32 + 8 * g : 0;
    const rt_bf16x8_t a = *reinterpret_cast<const rt_bf16x8_t *>(x + size_t(tok) * d + kk);
    // W_g piece: row ks*32 + lane/2, columns 8*(lane%2) .. +7 of the tile.
    const int row = ks * 32 + (lane >> 1);
    const int c0 = (lane & 1) * 8;
    const bool ok = row < d;
    const size_t ro = size_t(ok ? row : 0) * E + e0 + c0;
    uint4 wv;
    if (VEC) {
      wv = *reinterpret_cast<const uint4 *>(w + ro);
    } else {
      uint32_t t[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t lo = (c0 + 2 * c < ne) ? w[ro + 2 * c] : 0u;
        const uint32_t hi = (c0 + 2 * c + 1 < ne) ? w[ro + 2 * c + 1] : 0u;
        t[c] = lo | (hi << 16);
      }
      wv = make_uint4(t[0], t[1], t[2], t[3]);
    }
    *reinterpret_cast<uint4 *>(&sm.wl[wave][lane >> 1][c0]) = ok ? wv : make_uint4(0, 0, 0, 0);
    // Only this wave reads what it wrote; its LDS accesses run in order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    rt_bf16x8_t bfrag;
#pragma unroll
    for (int r = 0; r < 8; ++r) bfrag[r] = short(sm.wl[wave][8 * g + r][j]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfrag, acc, 0, 0, 0);
  }
  // acc holds rows 4g + i (tokens), column j (expert) of this wave's partial tile.
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.red[wave][4 * g + i][j] = acc[i];
  __syncthreads();
  float v = 0.0f;
  if (threadIdx.x < kRtTile * kRtTile) {
    const int ti = threadIdx.x / kRtTile, ej = threadIdx.x % kRtTile;
#pragma unroll
    for (int wv2 = 0; wv2 < kRtWaves; ++wv2) v += sm.red[wv2][ti][ej];
  }
  return v;
}

// Logit (t, e) completed from the slices' partial tiles in `part`
// ([tile][slices][256], tile = te + tiles_e * tt): bias[e], then the slices
// added in order. Loads are device-scope (other workgroups stored them) and
// up to eight are issued before the first is used.
__device__ __forceinline__ float router_logit(const float *__restrict__ part,
                                              const float *__restrict__ bias, int t, int e,
                                              int tiles_e, int slices) {
  const int tile = e / kRtTile + tiles_e * (t / kRtTile);
  float *tp = const_cast<float *>(part) + size_t(tile) * slices * (kRtTile * kRtTile) +
              (t % kRtTile) * kRtTile + (e % kRtTile);
  float v = bias ? bias[e] : 0.0f;
  for (int s0 = 0; s0 < slices; s0 += 8) {
    float p[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      p[q] = s0 + q < slices ? __hip_atomic_load(tp + (s0 + q) * (kRtTile * kRtTile), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (s0 + q < slices) v += p[q];
  }
  return v;
}

}  // namespace
}  // namespace moe
