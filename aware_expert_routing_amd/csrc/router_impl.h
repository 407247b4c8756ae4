// bf16 router tile ("Router Caching and Optimization", section "Analyzing
// Router Inference Cost", step 1: logits = x W_g + bias), as a device function
// run by one workgroup of 1024 threads (16 waves): the 16-token x 16-expert
// logit tile of blockIdx (x: experts, y: tokens) over the whole reduction, on
// MFMA (v_mfma_f32_16x16x32_bf16). Wave w takes the w-th sixteenth of the
// reduction; A fragments (8 consecutive features of one token) load straight
// from x; W_g's 16 columns are staged in LDS in blocks of 128 rows (16-byte
// loads, all issued before any is used) and read back as B fragments (8
// consecutive rows of one column). The waves' partial tiles are added in
// wave order, then the bias, so the logits are the same bits on every run
// and in every kernel that uses this function. They are stored with
// device-scope stores (another workgroup of the same kernel may read them).
#pragma once
#include "moe_internal.h"

namespace moe {
namespace {

typedef short rt_bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float rt_f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kRtThreads = 1024;
constexpr int kRtWaves = kRtThreads / 64;
constexpr int kRtTile = 16;     // tokens and experts per tile
constexpr int kRtBlock = 128;   // W_g rows per LDS block (4 k-steps)

struct RouterLds {
  uint16_t wl[kRtWaves][kRtBlock][kRtTile];  // per wave: W_g rows x 16 columns
  float red[kRtWaves][kRtTile][kRtTile];     // per wave: partial tile
};

// VEC: the tile's 16 columns are 16-byte aligned in every row (E % 16 == 0).
template <bool VEC>
__device__ __forceinline__ void router_tile(const uint16_t *__restrict__ x,
                                            const uint16_t *__restrict__ w,
                                            const float *__restrict__ bias, int B, int d, int E,
                                            float *__restrict__ logits, RouterLds &sm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * kRtTile, t0 = blockIdx.y * kRtTile;
  const int ne = min(kRtTile, E - e0);
  const int tok = min(t0 + j, B - 1);  // clamped: rows past B are computed and dropped
  const int nks = (d + 31) / 32;       // k-steps of 32 reduction rows
  const int per = (nks + kRtWaves - 1) / kRtWaves;
  const int ks0 = wave * per, ks1 = min(nks, ks0 + per);
  rt_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = ks0; kb < ks1; kb += 4) {
    rt_bf16x8_t a[4];
    uint4 wv[4];
    bool wok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // Features past d (or of k-steps this wave does not use) read feature
      // 0: any finite value does, the W_g rows they meet are zero.
      const int k = (kb + q) * 32 + 8 * g;
      const int kk = (kb + q < ks1 && k < d) ? k : 0;
      a[q] = *reinterpret_cast<const rt_bf16x8_t *>(x + size_t(tok) * d + kk);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int piece = lane + 64 * q;  // 256 pieces of 16 B: row piece/2, half piece%2
      const int row = kb * 32 + piece / 2;
      const int c0 = (piece & 1) * 8;
      // Rows past d read row 0 (every load in bounds, issued unconditionally)
      // and are stored as zero.
      const bool ok = row < d;
      wok[q] = ok;
      const size_t ro = size_t(ok ? row : 0) * E + e0 + c0;
      if (VEC) {
        wv[q] = *reinterpret_cast<const uint4 *>(w + ro);
      } else {
        uint32_t t[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t lo = (c0 + 2 * c < ne) ? w[ro + 2 * c] : 0u;
          const uint32_t hi = (c0 + 2 * c + 1 < ne) ? w[ro + 2 * c + 1] : 0u;
          t[c] = lo | (hi << 16);
        }
        wv[q] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int piece = lane + 64 * q;
      *reinterpret_cast<uint4 *>(&sm.wl[wave][piece / 2][(piece & 1) * 8]) =
          wok[q] ? wv[q] : make_uint4(0, 0, 0, 0);
    }
    // Only this wave reads what it wrote; its LDS accesses run in order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (kb + q < ks1) {
        rt_bf16x8_t bfrag;
#pragma unroll
        for (int r = 0; r < 8; ++r) bfrag[r] = short(sm.wl[wave][q * 32 + 8 * g + r][j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], bfrag, acc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // acc holds rows 4g + i (tokens), column j (expert) of this wave's partial tile.
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.red[wave][4 * g + i][j] = acc[i];
  __syncthreads();
  if (threadIdx.x < kRtTile * kRtTile) {
    const int ti = threadIdx.x / kRtTile, ej = threadIdx.x % kRtTile;
    if (t0 + ti < B && ej < ne) {
      float v = bias ? bias[e0 + ej] : 0.0f;
#pragma unroll
      for (int wv2 = 0; wv2 < kRtWaves; ++wv2) v += sm.red[wv2][ti][ej];
      __hip_atomic_store(logits + size_t(t0 + ti) * E + e0 + ej, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace
}  // namespace moe
