// Grouped SwiGLU expert FFN over the batch's active experts:
//   y[t] = sum_j w[t,j] * (SiLU(x_t G_e) * (x_t U_e)) D_e,  e = slot j's expert,
// reading only the weights of experts in the active list ("Lynx", Technical
// Summary 1: decode latency follows the number of distinct experts loaded;
// "Opportunistic Expert Activation", abstract: MoE latency is governed by the
// number of activated experts).
//
// bf16 path (the bandwidth-bound one):
//   up      one work item = (active expert, 64-column strip of I, slice of d).
//           Weight tiles of G and U stream HBM -> registers (two stages ahead)
//           -> LDS, where 16-byte chunks are XOR-swizzled so that the 16-bit
//           reads along the reduction dimension are bank-conflict free. The
//           transposed fragments feed either v_mfma_f32_16x16x32_bf16 (tokens
//           of the expert as the 16-row A operand) or, for experts with few
//           tokens, wave-level v_dot2_f32_bf16 dot products. Partial sums per
//           slice go to the workspace (float32).
//   h       h = SiLU(sum_s g_s) * (sum_s u_s), summed in slice order, stored
//           as bf16 (round to nearest even).
//   down    one work item = (active expert, 64-column strip of d), whole I;
//           same tile pipeline over D, A operand = the expert's h rows.
//           Each output row is scaled by its gate weight and written to
//           part[t][j][:].
//   combine y[t] = sum over slots j in order of part[t][j] (deterministic;
//           no float atomics), rounded to bf16.
// float32 path (small layers): direct per-output dot products.
#include "moe_internal.h"

namespace moe {
namespace {

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x2_t __attribute__((__vector_size__(2 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk

constexpr int kThreads = 256;   // 4 waves
constexpr int kChunks = 8;      // 16-byte chunks per 64-column tile row
constexpr int kMaxTok = 64;     // tokens per pass over an item's weights
constexpr int kMaxMT = kMaxTok / 16;
constexpr int kDotMaxT = 4;     // experts with <= this many tokens use dot2
constexpr int kGridCap = 2048;
static_assert(kStripCols == 64 && kStageRows == 64, "tile constants");

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Physical chunk of logical chunk c in weight-tile row r. Rows 8 apart (the
// four k-blocks a fragment read touches) land on disjoint chunk pairs.
__device__ __forceinline__ int swz_w(int r, int c) { return c ^ (((r >> 3) & 3) << 1); }
// Physical chunk of logical chunk c in activation-tile row m.
__device__ __forceinline__ int swz_x(int m, int c) { return c ^ (m & 7); }

template <int NMAT>
struct Tiles {
  u32x4_t w[2][NMAT][kStageRows][kChunks];
  u32x4_t x[2][kMaxTok][kChunks];
};

template <int NMAT>
struct StageRegs {
  u32x4_t w[NMAT][2];
  u32x4_t x[2];
};

// One pass of a work item: C[Tp, 64] (+)= A[Tp, nrows] * W[nrows, 64] for
// NMAT weight matrices sharing A.
template <int NMAT>
struct ItemPass {
  const uint16_t *w[NMAT];  // first row of the slice, column 0 of the matrix
  int ld;                   // row stride of W (elements) = its column count
  int nrows;                // reduction length of the slice (multiple of 8)
  int col0;                 // first column of the strip
  const uint16_t *arow[2];  // A rows staged by this thread (always a valid row)
  bool arow_ok[2];          // false: stage a zero row instead
  int T;                    // tokens in this pass, 1..kMaxTok
};

// Loads are unconditional from an address that is always valid (the tile's
// first element when the wanted one is out of range); out-of-range chunks are
// zeroed by selecting on the loaded value, which keeps every load a plain
// global_load_dwordx4 with no branch.
template <int NMAT>
__device__ __forceinline__ void load_stage(const ItemPass<NMAT> &p, int st, StageRegs<NMAT> &R) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int r = idx >> 3, c = idx & 7;
    const int row = st * kStageRows + r;
    const int col = p.col0 + 8 * c;
    const bool ok = row < p.nrows && col < p.ld;
    const size_t off = ok ? size_t(row) * p.ld + col : 0;
    const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
      R.w[mat][i] = *reinterpret_cast<const u32x4_t *>(p.w[mat] + off) & keep;
    const int k = st * kStageRows + 8 * c;
    const bool okx = p.arow_ok[i] && k < p.nrows;
    const uint32_t keepx = okx ? 0xFFFFFFFFu : 0u;
    R.x[i] = *reinterpret_cast<const u32x4_t *>(p.arow[i] + (okx ? k : 0)) & keepx;
  }
}

template <int NMAT>
__device__ __forceinline__ void store_stage(Tiles<NMAT> &sm, int buf, const StageRegs<NMAT> &R) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int r = idx >> 3, c = idx & 7;
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) sm.w[buf][mat][r][swz_w(r, c)] = R.w[mat][i];
    sm.x[buf][r][swz_x(r, c)] = R.x[i];
  }
}

// Accumulators of one pass. MFMA: acc[mat][mt] holds rows 4*(lane/16)+i of
// M-tile mt, column 16*wave + lane%16. Dot: accd[mat][m] holds token m's
// partial dot product over this lane's k-blocks.
template <int NMAT>
struct Acc {
  f32x4_t acc[NMAT][kMaxMT];
  float accd[NMAT][kDotMaxT];
};

template <int NMAT>
__device__ __forceinline__ void compute_stage(const Tiles<NMAT> &sm, int buf, int T, bool dot,
                                     Acc<NMAT> &A) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int n16 = lane & 15;
  const int nmt = (T + 15) >> 4;
#pragma unroll
  for (int kk = 0; kk < kStageRows; kk += 32) {
    const int r0 = kk + 8 * q;
    const int pc = swz_w(r0, 2 * wave + (n16 >> 3));
    bf16x8_t b[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
      const uint16_t *src = reinterpret_cast<const uint16_t *>(&sm.w[buf][mat][r0][pc]) + (n16 & 7);
#pragma unroll
      for (int j = 0; j < 8; ++j) b[mat][j] = short(src[j * kChunks * 8]);
    }
    const int xc = (kk >> 3) + q;
    if (!dot) {
#pragma unroll
      for (int mt = 0; mt < kMaxMT; ++mt) {
        if (mt < nmt) {
          const int m = 16 * mt + n16;
          const u32x4_t av = sm.x[buf][m][swz_x(m, xc)];
          bf16x8_t a;
          __builtin_memcpy(&a, &av, sizeof(a));
#pragma unroll
          for (int mat = 0; mat < NMAT; ++mat)
            A.acc[mat][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[mat], A.acc[mat][mt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < kDotMaxT; ++m) {
        if (m < T) {
          const u32x4_t av = sm.x[buf][m][swz_x(m, xc)];
          const uint32_t xa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int mat = 0; mat < NMAT; ++mat) {
            float s = A.accd[mat][m];
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              bf16x2_t wv, xv;
              wv[0] = b[mat][2 * pp];
              wv[1] = b[mat][2 * pp + 1];
              __builtin_memcpy(&xv, &xa[pp], sizeof(xv));
              s = __builtin_amdgcn_fdot2_f32_bf16(wv, xv, s, false);
            }
            A.accd[mat][m] = s;
          }
        }
      }
    }
  }
}

// Streams the pass's weight rows through the LDS pipeline and accumulates.
template <int NMAT>
__device__ __forceinline__ void run_pass(Tiles<NMAT> &sm, const ItemPass<NMAT> &p, bool dot, Acc<NMAT> &A) {
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
#pragma unroll
    for (int mt = 0; mt < kMaxMT; ++mt) A.acc[mat][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kDotMaxT; ++m) A.accd[mat][m] = 0.f;
  }
  const int nst = (p.nrows + kStageRows - 1) / kStageRows;
  StageRegs<NMAT> R0, R1;
  load_stage(p, 0, R0);
  if (nst > 1) load_stage(p, 1, R1);
  __syncthreads();  // the previous pass may still read the LDS tiles
  for (int st = 0; st < nst; st += 2) {
    store_stage(sm, 0, R0);
    __syncthreads();
    if (st + 2 < nst) load_stage(p, st + 2, R0);
    compute_stage(sm, 0, p.T, dot, A);
    if (st + 1 >= nst) break;
    store_stage(sm, 1, R1);
    __syncthreads();
    if (st + 3 < nst) load_stage(p, st + 3, R1);
    compute_stage(sm, 1, p.T, dot, A);
  }
  if (dot) {
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
      for (int m = 0; m < kDotMaxT; ++m) {
        float v = A.accd[mat][m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        A.accd[mat][m] = v;
      }
  }
}

// ------------------------------------------------------------------- up
__global__ __launch_bounds__(kThreads) void up_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg, const uint16_t *__restrict__ wu,
    int d, int I, int P, const int32_t *__restrict__ n_active, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_token, int nks,
    int slice_rows, float *__restrict__ gpart) {
  __shared__ Tiles<2> sm;
  const int nstrip = (I + kStripCols - 1) / kStripCols;
  const int per_expert = nstrip * nks;
  const int items = n_active[0] * per_expert;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, n16 = lane & 15;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int a = item / per_expert;
    const int rem = item - a * per_expert;
    const int strip = rem / nks;
    const int ks = rem - strip * nks;
    const int e = active[a];
    const int p0 = offsets[a];
    const int T = offsets[a + 1] - p0;
    const int row0 = ks * slice_rows;
    ItemPass<2> p;
    p.ld = I;
    p.nrows = min(slice_rows, d - row0);
    p.col0 = strip * kStripCols;
    p.w[0] = wg + (size_t(e) * d + row0) * I;
    p.w[1] = wu + (size_t(e) * d + row0) * I;
    const int col = p.col0 + 16 * wave + n16;
    for (int t0 = 0; t0 < T; t0 += kMaxTok) {
      p.T = min(kMaxTok, T - t0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = (threadIdx.x + kThreads * i) >> 3;
        p.arow_ok[i] = m < p.T;
        p.arow[i] = x + size_t(pair_token[p0 + t0 + (m < p.T ? m : 0)]) * d + row0;
      }
      const bool dot = p.T <= kDotMaxT;
      Acc<2> A;
      run_pass(sm, p, dot, A);
      if (col >= I) continue;
      if (!dot) {
#pragma unroll
        for (int mt = 0; mt < kMaxMT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * q + i;
            if (m < p.T) {
#pragma unroll
              for (int mat = 0; mat < 2; ++mat)
                gpart[((size_t(ks) * 2 + mat) * P + p0 + t0 + m) * I + col] = A.acc[mat][mt][i];
            }
          }
      } else if (q == 0) {
#pragma unroll
        for (int m = 0; m < kDotMaxT; ++m)
          if (m < p.T) {
#pragma unroll
            for (int mat = 0; mat < 2; ++mat)
              gpart[((size_t(ks) * 2 + mat) * P + p0 + t0 + m) * I + col] = A.accd[mat][m];
          }
      }
    }
  }
}

// -------------------------------------------------------------------- h
// One thread per 4 consecutive columns of one pair.
__global__ __launch_bounds__(kThreads) void h_kernel(const float *__restrict__ gpart, int nks,
                                                     int P, int I, const int32_t *__restrict__ n_active,
                                                     const int32_t *__restrict__ offsets,
                                                     uint16_t *__restrict__ h) {
  const int total = offsets[n_active[0]];
  const int q4 = I / 4;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total * q4) return;
  const int pr = idx / q4;
  const int c = (idx - pr * q4) * 4;
  float4 g = make_float4(0, 0, 0, 0), u = make_float4(0, 0, 0, 0);
  for (int s = 0; s < nks; ++s) {
    const float4 gv = *reinterpret_cast<const float4 *>(gpart + ((size_t(s) * 2 + 0) * P + pr) * I + c);
    const float4 uv = *reinterpret_cast<const float4 *>(gpart + ((size_t(s) * 2 + 1) * P + pr) * I + c);
    g.x += gv.x; g.y += gv.y; g.z += gv.z; g.w += gv.w;
    u.x += uv.x; u.y += uv.y; u.z += uv.z; u.w += uv.w;
  }
  ushort4 o;
  o.x = f32_to_bf16(silu(g.x) * u.x);
  o.y = f32_to_bf16(silu(g.y) * u.y);
  o.z = f32_to_bf16(silu(g.z) * u.z);
  o.w = f32_to_bf16(silu(g.w) * u.w);
  *reinterpret_cast<ushort4 *>(h + size_t(pr) * I + c) = o;
}

// ----------------------------------------------------------------- down
__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ wd, int d, int I, int k,
    const int32_t *__restrict__ n_active, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_token,
    const int32_t *__restrict__ pair_slot, const float *__restrict__ topk_w,
    float *__restrict__ part) {
  __shared__ Tiles<1> sm;
  const int nstrip = (d + kStripCols - 1) / kStripCols;
  const int items = n_active[0] * nstrip;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, n16 = lane & 15;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int a = item / nstrip;
    const int strip = item - a * nstrip;
    const int e = active[a];
    const int p0 = offsets[a];
    const int T = offsets[a + 1] - p0;
    ItemPass<1> p;
    p.ld = d;
    p.nrows = I;
    p.col0 = strip * kStripCols;
    p.w[0] = wd + size_t(e) * I * d;
    const int col = p.col0 + 16 * wave + n16;
    for (int t0 = 0; t0 < T; t0 += kMaxTok) {
      p.T = min(kMaxTok, T - t0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = (threadIdx.x + kThreads * i) >> 3;
        p.arow_ok[i] = m < p.T;
        p.arow[i] = h + size_t(p0 + t0 + (m < p.T ? m : 0)) * I;
      }
      const bool dot = p.T <= kDotMaxT;
      Acc<1> A;
      run_pass(sm, p, dot, A);
      if (col >= d) continue;
      if (!dot) {
#pragma unroll
        for (int mt = 0; mt < kMaxMT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * mt + 4 * q + i;
            if (m < p.T) {
              const int pr = p0 + t0 + m;
              const int slot = pair_token[pr] * k + pair_slot[pr];
              part[size_t(slot) * d + col] = topk_w[slot] * A.acc[0][mt][i];
            }
          }
      } else if (q == 0) {
#pragma unroll
        for (int m = 0; m < kDotMaxT; ++m)
          if (m < p.T) {
            const int pr = p0 + t0 + m;
            const int slot = pair_token[pr] * k + pair_slot[pr];
            part[size_t(slot) * d + col] = topk_w[slot] * A.accd[0][m];
          }
      }
    }
  }
}

// -------------------------------------------------------------- combine
template <typename OutT>
__device__ __forceinline__ void store4(OutT *y, float4 v);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t *y, float4 v) {
  ushort4 o;
  o.x = f32_to_bf16(v.x);
  o.y = f32_to_bf16(v.y);
  o.z = f32_to_bf16(v.z);
  o.w = f32_to_bf16(v.w);
  *reinterpret_cast<ushort4 *>(y) = o;
}
template <>
__device__ __forceinline__ void store4<float>(float *y, float4 v) {
  *reinterpret_cast<float4 *>(y) = v;
}

template <typename OutT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ part,
                                                           const int32_t *__restrict__ topk_ids,
                                                           int B, int d, int k, OutT *__restrict__ y) {
  const int q4 = d / 4;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= B * q4) return;
  const int t = idx / q4;
  const int c = (idx - t * q4) * 4;
  float4 acc = make_float4(0, 0, 0, 0);
  for (int j = 0; j < k; ++j) {
    if (topk_ids[t * k + j] < 0) continue;
    const float4 v = *reinterpret_cast<const float4 *>(part + (size_t(t) * k + j) * d + c);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  store4<OutT>(y + size_t(t) * d + c, acc);
}

// ----------------------------------------------------------- float32 path
// One thread per (pair, column of I): h = SiLU(x G) * (x U), float32.
__global__ __launch_bounds__(kThreads) void up_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wg, const float *__restrict__ wu, int d,
    int I, int k, const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_token, const int32_t *__restrict__ pair_slot,
    const int32_t *__restrict__ topk_ids, float *__restrict__ h) {
  const int total = offsets[n_active[0]];
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total * I) return;
  const int pr = idx / I, c = idx - pr * I;
  const int t = pair_token[pr];
  const int e = topk_ids[t * k + pair_slot[pr]];
  const float *xr = x + size_t(t) * d;
  const float *G = wg + size_t(e) * d * I + c;
  const float *U = wu + size_t(e) * d * I + c;
  float g = 0.f, u = 0.f;
  for (int i = 0; i < d; ++i) {
    g = fmaf(xr[i], G[size_t(i) * I], g);
    u = fmaf(xr[i], U[size_t(i) * I], u);
  }
  h[size_t(pr) * I + c] = silu(g) * u;
}

// One thread per (pair, column of d): part = w * (h D), float32.
__global__ __launch_bounds__(kThreads) void down_f32_kernel(
    const float *__restrict__ h, const float *__restrict__ wd, int d, int I, int k,
    const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_token, const int32_t *__restrict__ pair_slot,
    const int32_t *__restrict__ topk_ids, const float *__restrict__ topk_w,
    float *__restrict__ part) {
  const int total = offsets[n_active[0]];
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total * d) return;
  const int pr = idx / d, c = idx - pr * d;
  const int slot = pair_token[pr] * k + pair_slot[pr];
  const int e = topk_ids[slot];
  const float *hr = h + size_t(pr) * I;
  const float *D = wd + size_t(e) * I * d + c;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(hr[i], D[size_t(i) * d], acc);
  part[size_t(slot) * d + c] = topk_w[slot] * acc;
}

}  // namespace

hipError_t launch_expert_ffn(const void *x, const void *w_gate, const void *w_up,
                             const void *w_down, moe_dtype_t dt, int B, int d, int E, int I,
                             int k, const moe_routing_t &r, void *y, char *ws,
                             const Workspace &plan, hipStream_t s) {
  const int P = B * k;
  const int max_active = E < P ? E : P;
  float *part = reinterpret_cast<float *>(ws + plan.down_part);
  if (dt == MOE_BF16) {
    float *gpart = reinterpret_cast<float *>(ws + plan.up_part);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + plan.h);
    const int up_items = max_active * ceil_div(I, kStripCols) * plan.up_slices;
    up_kernel<<<up_items < kGridCap ? up_items : kGridCap, kThreads, 0, s>>>(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_gate),
        static_cast<const uint16_t *>(w_up), d, I, P, r.n_active, r.active_experts,
        r.expert_offsets, r.pair_token, plan.up_slices, plan.up_slice_rows, gpart);
    h_kernel<<<ceil_div(P * (I / 4), kThreads), kThreads, 0, s>>>(gpart, plan.up_slices, P, I,
                                                                 r.n_active, r.expert_offsets, h);
    const int down_items = max_active * ceil_div(d, kStripCols);
    down_kernel<<<down_items < kGridCap ? down_items : kGridCap, kThreads, 0, s>>>(
        h, static_cast<const uint16_t *>(w_down), d, I, k, r.n_active, r.active_experts,
        r.expert_offsets, r.pair_token, r.pair_slot, r.topk_w, part);
    combine_kernel<uint16_t><<<ceil_div(B * (d / 4), kThreads), kThreads, 0, s>>>(
        part, r.topk_ids, B, d, k, static_cast<uint16_t *>(y));
  } else {
    float *h = reinterpret_cast<float *>(ws + plan.h);
    up_f32_kernel<<<ceil_div(P * I, kThreads), kThreads, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(w_gate),
        static_cast<const float *>(w_up), d, I, k, r.n_active, r.expert_offsets, r.pair_token,
        r.pair_slot, r.topk_ids, h);
    down_f32_kernel<<<ceil_div(P * d, kThreads), kThreads, 0, s>>>(
        h, static_cast<const float *>(w_down), d, I, k, r.n_active, r.expert_offsets,
        r.pair_token, r.pair_slot, r.topk_ids, r.topk_w, part);
    combine_kernel<float><<<ceil_div(B * (d / 4), kThreads), kThreads, 0, s>>>(
        part, r.topk_ids, B, d, k, static_cast<float *>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
