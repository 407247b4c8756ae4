// Grouped SwiGLU expert FFN over the batch's active experts:
//   y[t] = sum_j w[t,j] * (SiLU(x_t G_e) * (x_t U_e)) D_e,  e = slot j's expert,
// reading only the weights of experts in the active list ("Lynx", Technical
// Summary 1: decode latency follows the number of distinct experts loaded;
// "Opportunistic Expert Activation", abstract: MoE latency is governed by the
// number of activated experts).
//
// bf16 path. Both products (gate/up: A = x, W = G and U; down: A = h, W = D)
// run through one persistent streaming kernel:
//   * a work item is one active expert x one 64-column strip of the output x
//     one slice of the reduction; a workgroup takes items b, b+G, b+2G, ...;
//   * the workgroup's items form one flat sequence of 64-row stages; stages
//     are copied HBM -> LDS by buffer_load ... lds (no registers involved) into
//     a ring of slots, several stages ahead of the one being used, so the copy
//     of the next item's weights overlaps the end of the current one;
//   * each wave counts the copies it has issued and waits with s_waitcnt
//     vmcnt(n) for exactly the stage it needs, then one s_barrier;
//   * weight rows are stored with their 16-byte chunks XOR-swizzled so that
//     the transposing LDS reads (ds_read_b64_tr_b16) that build MFMA B
//     fragments along the reduction dimension are bank-conflict free;
//   * an expert's tokens form the A operand (16 rows per MFMA tile,
//     v_mfma_f32_16x16x32_bf16). Experts with at most kDotMaxT tokens use
//     wave-level v_dot2_f32_bf16 dot products on the same fragments instead.
// Gate/up partial sums per slice and down-projection outputs per (token, slot)
// go to the workspace; small kernels finish the SwiGLU (h) and the weighted,
// fixed-order combine over slots (no float atomics).
// float32 path (small layers): direct per-output dot products.
#include "moe_internal.h"

namespace moe {
namespace {

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef short bf16x2_t __attribute__((__vector_size__(2 * sizeof(short))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;                   // 4 waves; wave w owns columns 16w..16w+15
constexpr int kBK = kStageRows;                 // reduction rows per stage
constexpr int kKSteps = kBK / 32;               // MFMA k-steps per stage
constexpr int kRowBytes = kStripCols * 2;       // one strip row of bf16
constexpr int kWTile = kBK * kRowBytes;         // bytes of one weight matrix per stage
constexpr int kMaxTok = 64;                     // tokens per pass (4 MFMA row tiles)
constexpr int kDotMaxT = 4;                     // experts with <= this many tokens use dot2
constexpr int kMaxPairs = kMaxB * kMaxK;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, gfx9 data format
constexpr int kLdsBytes = 160 * 1024;
static_assert(kStripCols == 64 && kBK == 128, "tile constants");

// Routing lists staged in LDS once per workgroup (the loop reads them with
// the inline-assembly helpers below).
constexpr int kMetaTok = 0;                            // uint8 token of each pair
constexpr int kMetaAct = kMetaTok + kMaxPairs;         // int16 active expert list
constexpr int kMetaOff = kMetaAct + 2 * kMaxE;         // int16 CSR offsets
constexpr int kMetaBytes = kMetaOff + 2 * (kMaxE + 1) + 14;

// LDS plan of one instantiation. A stage slot holds NMAT weight tiles
// [kBK rows][64 columns] and the A tile, stored per k-step as
// [kKSteps][16*MTX rows][64 bytes] so that every lane's fragment address is a
// per-lane constant plus a compile-time offset.
template <int NMAT, int MTX>
struct Shape {
  static constexpr int kXSub = 16 * MTX * 64;
  static constexpr int kXTile = kKSteps * kXSub;
  static constexpr int kSlot = NMAT * kWTile + kXTile;
  static constexpr int kStages = (kLdsBytes - kMetaBytes) / kSlot;
  static constexpr int kCopies = 4 * NMAT + MTX;  // 1 KB copies per wave per stage
  static_assert(kStages >= 3, "too few stages");
  static_assert((kStages - 2) * kCopies <= 63, "vmcnt range");
};

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// XOR applied to the 16-byte chunk index of weight row r of a stage. The
// transposing reads of one instruction touch rows kk + 8g + 4h + {0..3}
// (g = 0..3); this map spreads their chunk pairs over the banks, and it does
// not depend on kk (a multiple of 32), so a lane's read offsets are constants.
__device__ __forceinline__ int swz_w(int r) { return (((r >> 1) ^ (r >> 3)) & 3) << 1; }
// Chunk XOR of A-tile row m (rows of 64 bytes = 4 chunks): the 16 rows a
// fragment reads at one logical chunk hit 16 distinct 4-bank groups.
__device__ __forceinline__ int swz_x(int m) { return (m >> 2) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kRsrcWord3);
}

// Copies 16 bytes per lane from buffer offset voff + soff into LDS at
// dst + 16*lane. Offsets at or past the end of the buffer read as zero.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff,
                                      uint32_t soff) {
  // A C-style cast is the way to move a generic pointer into the LDS address space.
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst), 16, int(voff), int(soff), 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier. Compiler barriers keep LDS
// accesses on their side of the s_barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  constexpr int enc = (N & 15) | ((N >> 4) << 14) | (7 << 4);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(enc);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_void_t *)(p)));
}

// LDS reads as inline assembly that waits for its own results (lgkmcnt(0))
// before returning: the compiler then sees no LDS load in the loop and adds
// no wait on the stage copies in flight, whose completion the loop tracks
// itself with s_waitcnt vmcnt.
__device__ __forceinline__ int lds_u8(uint32_t a) {
  int v;
  asm volatile("ds_read_u8 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ int lds_i16(uint32_t a) {
  int v;
  asm volatile("ds_read_i16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a));
  return v;
}

__device__ __forceinline__ void lds_tr2(uint32_t a0, uint32_t a1, bf16x8_t &b) {
  long lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\t"
               "ds_read_b64_tr_b16 %1, %3\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(lo), "=&v"(hi)
               : "v"(a0), "v"(a1));
  __builtin_memcpy(&b, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char *>(&b) + 8, &hi, 8);
}

__device__ __forceinline__ void lds_tr4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                        bf16x8_t &b0, bf16x8_t &b1) {
  long v0, v1, v2, v3;
  asm volatile("ds_read_b64_tr_b16 %0, %4\n\t"
               "ds_read_b64_tr_b16 %1, %5\n\t"
               "ds_read_b64_tr_b16 %2, %6\n\t"
               "ds_read_b64_tr_b16 %3, %7\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
               : "v"(a0), "v"(a1), "v"(a2), "v"(a3));
  __builtin_memcpy(&b0, &v0, 8);
  __builtin_memcpy(reinterpret_cast<char *>(&b0) + 8, &v1, 8);
  __builtin_memcpy(&b1, &v2, 8);
  __builtin_memcpy(reinterpret_cast<char *>(&b1) + 8, &v3, 8);
}

template <int NA>
__device__ __forceinline__ void lds_b128(const uint32_t (&a)[4], bf16x8_t (&x)[4]);
template <>
__device__ __forceinline__ void lds_b128<1>(const uint32_t (&a)[4], bf16x8_t (&x)[4]) {
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x[0]) : "v"(a[0]));
}
template <>
__device__ __forceinline__ void lds_b128<2>(const uint32_t (&a)[4], bf16x8_t (&x)[4]) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]) : "v"(a[0]), "v"(a[1]));
}
template <>
__device__ __forceinline__ void lds_b128<3>(const uint32_t (&a)[4], bf16x8_t (&x)[4]) {
  asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]));
}
template <>
__device__ __forceinline__ void lds_b128<4>(const uint32_t (&a)[4], bf16x8_t (&x)[4]) {
  asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
               "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
               : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

struct Params {
  const uint16_t *A;       // x [B,d] (up) or h [P,I] (down)
  uint32_t a_bytes;        // size of A in bytes
  int a_ld;                // row stride of A (elements): d (up) or I (down)
  const uint16_t *W[2];    // G, U (up) or D (down): [E, K, N]
  int K, N;                // reduction length and output columns per expert
  int slices, slice_rows;  // reduction slices per expert
  int P;                   // pair capacity (B*k)
  float *out;              // up: float [slices][2][P][N]; down: float [P][N] by pair
};

// A position in a workgroup's stage sequence. All fields are wave-uniform
// except arow (the A rows this lane copies).
struct Cursor {
  int item, n_items, per_expert;
  int e, p0, T, strip, ks, row0, nrows, nst, npass;
  int pass, kst;
  bool valid;
};

template <int NMAT, int MTX, bool UP>
struct Stream {
  using S = Shape<NMAT, MTX>;
  const Params &p;
  uint32_t meta;            // LDS address of the routing lists
  int wave, lane, g, j;
  uint32_t wvoff[4];        // weight copy offsets (bytes) within a stage, copies w + 4h
  uint32_t trc[2];          // transposing-read offsets within a weight tile
  uint32_t xrd;             // A-fragment read offset within a k-step sub-tile
  uint32_t dotrd;           // token-row read offset for the dot2 path

  __device__ __forceinline__ Stream(const Params &pp, uint32_t meta_addr) : p(pp), meta(meta_addr) {
    wave = wave_id();
    lane = threadIdx.x & 63;
    g = lane >> 4;
    j = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = 8 * (wave + 4 * h) + (lane >> 3);
      const int lc = (lane & 7) ^ swz_w(r);
      wvoff[h] = uint32_t(r) * uint32_t(p.N) * 2u + uint32_t(lc) * 16u;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R = 8 * g + 4 * h + (j >> 2);
      const int c = 2 * wave + ((j & 3) >> 1);
      trc[h] = uint32_t(R * kRowBytes + ((c ^ swz_w(R)) << 4) + ((j & 1) << 3));
    }
    xrd = uint32_t(j * 64 + ((g ^ swz_x(j)) << 4));
    dotrd = uint32_t(g << 4);
  }

  __device__ __forceinline__ void decode(Cursor &c) const {
    c.valid = c.item < c.n_items;
    if (!c.valid) return;
    const int a = c.item / c.per_expert;
    const int rem = c.item - a * c.per_expert;
    c.strip = rem / p.slices;
    c.ks = rem - c.strip * p.slices;
    c.e = __builtin_amdgcn_readfirstlane(lds_i16(meta + kMetaAct + 2 * a));
    c.p0 = __builtin_amdgcn_readfirstlane(lds_i16(meta + kMetaOff + 2 * a));
    c.T = __builtin_amdgcn_readfirstlane(lds_i16(meta + kMetaOff + 2 * a + 2)) - c.p0;
    c.row0 = c.ks * p.slice_rows;
    c.nrows = min(p.slice_rows, p.K - c.row0);
    c.nst = (c.nrows + kBK - 1) / kBK;
    c.npass = (c.T + kMaxTok - 1) / kMaxTok;
    c.pass = 0;
    c.kst = 0;
  }
  __device__ __forceinline__ void advance(Cursor &c, int stride) const {
    if (++c.kst < c.nst) return;
    c.kst = 0;
    if (++c.pass < c.npass) return;
    c.item += stride;
    decode(c);
  }
  __device__ __forceinline__ static int tp(const Cursor &c) { return min(kMaxTok, c.T - c.pass * kMaxTok); }

  // Byte offset of the A row this lane copies for its copy h (MTX copies per
  // wave, one 16-row tile each, all at k-step `wave` of the stage).
  __device__ __forceinline__ uint32_t xvoff(const Cursor &c, int h) const {
    const int m = 16 * h + (lane >> 2);
    const int T = tp(c);
    const int pr = c.p0 + c.pass * kMaxTok + (m < T ? m : T - 1);
    const int arow = UP ? lds_u8(meta + kMetaTok + pr) : pr;
    const int lc = (lane & 3) ^ swz_x(m);
    return (uint32_t(arow) * uint32_t(p.a_ld) + uint32_t(wave * 32 + lc * 8)) * 2u;
  }

  // Issues the copies of stage c into `slot` (S::kCopies per wave).
  __device__ __forceinline__ void issue(const Cursor &c, unsigned char *slot) const {
    const size_t base = (size_t(c.e) * p.K + c.row0) * p.N;
    const uint32_t wbytes = uint32_t(c.nrows) * uint32_t(p.N) * 2u;
    const uint32_t soff = (uint32_t(c.kst * kBK) * uint32_t(p.N) + uint32_t(c.strip * kStripCols)) * 2u;
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p.W[mat] + base, wbytes);
#pragma unroll
      for (int h = 0; h < 4; ++h) dma16(r, slot + mat * kWTile + (wave + 4 * h) * 1024, wvoff[h], soff);
    }
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
    const uint32_t xsoff = uint32_t(c.row0 + c.kst * kBK) * 2u;
#pragma unroll
    for (int h = 0; h < MTX; ++h)
      dma16(ra, slot + NMAT * kWTile + wave * S::kXSub + h * 1024, xvoff(c, h), xsoff);
  }
};

template <int NMAT>
struct Acc {
  f32x4_t mf[NMAT][4];        // MFMA: rows 4*(lane/16)+i of tile mt, column 16*wave + lane%16
  float dot[NMAT][kDotMaxT];  // dot2: token m over this lane's k-groups
};

template <int NMAT>
__device__ __forceinline__ void clear(Acc<NMAT> &acc) {
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc.mf[mat][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kDotMaxT; ++m) acc.dot[mat][m] = 0.f;
  }
}

// B fragments of k-step ks for this lane: column 16*wave + j, rows
// 32ks + 8g .. 32ks + 8g + 7 of each weight tile. The transposing read gives
// lane j of a 16-lane group element j of the four rows its group's lanes point
// at (lane 4r+q points at row r, columns 4q..4q+3).
template <int NMAT>
__device__ __forceinline__ void b_frags(uint32_t slot, const uint32_t (&trc)[2], int ks,
                                        bf16x8_t (&b)[2]) {
  const uint32_t o = slot + uint32_t(ks * 32 * kRowBytes);
  if (NMAT == 2)
    lds_tr4(o + trc[0], o + trc[1], o + kWTile + trc[0], o + kWTile + trc[1], b[0], b[1]);
  else
    lds_tr2(o + trc[0], o + trc[1], b[0]);
}

template <int NMAT, int MTX, int NA>
__device__ __forceinline__ void mfma_stage(uint32_t slot, uint32_t xslot, const uint32_t (&trc)[2],
                                           uint32_t xrd, Acc<NMAT> &acc) {
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    bf16x8_t b[2];
    b_frags<NMAT>(slot, trc, ks, b);
    uint32_t aa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) aa[mt] = xslot + uint32_t(ks * Shape<NMAT, MTX>::kXSub + mt * 1024) + xrd;
    bf16x8_t a[4];
    lds_b128<NA>(aa, a);
#pragma unroll
    for (int mt = 0; mt < NA; ++mt)
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat)
        acc.mf[mat][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[mat], acc.mf[mat][mt], 0, 0, 0);
  }
}

template <int NMAT, int MTX>
__device__ __forceinline__ void dot_stage(uint32_t slot, uint32_t xslot, const uint32_t (&trc)[2],
                                          uint32_t dotrd, int T, Acc<NMAT> &acc) {
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    bf16x8_t b[2];
    b_frags<NMAT>(slot, trc, ks, b);
    // Rows 0..3 of the k-step's A sub-tile: token m's 8 values of this lane's
    // k-group (rows below 4 are not swizzled).
    const uint32_t xb = xslot + uint32_t(ks * Shape<NMAT, MTX>::kXSub) + dotrd;
    const uint32_t aa[4] = {xb, xb + 64, xb + 128, xb + 192};
    bf16x8_t a[4];
    lds_b128<4>(aa, a);
#pragma unroll
    for (int m = 0; m < kDotMaxT; ++m) {
      if (m < T) {
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) {
          float s = acc.dot[mat][m];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x2_t wv, xv;
            wv[0] = b[mat][2 * q];
            wv[1] = b[mat][2 * q + 1];
            xv[0] = a[m][2 * q];
            xv[1] = a[m][2 * q + 1];
            s = __builtin_amdgcn_fdot2_f32_bf16(wv, xv, s, false);
          }
          acc.dot[mat][m] = s;
        }
      }
    }
  }
}

template <int NMAT, int MTX>
__device__ __forceinline__ void compute_stage(uint32_t slot, const uint32_t (&trc)[2], uint32_t xrd,
                                              uint32_t dotrd, int T, Acc<NMAT> &acc) {
  const uint32_t xslot = slot + NMAT * kWTile;
  if (T <= kDotMaxT) {
    dot_stage<NMAT, MTX>(slot, xslot, trc, dotrd, T, acc);
    return;
  }
  const int na = (T + 15) >> 4;
  if (MTX == 1 || na == 1) mfma_stage<NMAT, MTX, 1>(slot, xslot, trc, xrd, acc);
  else if (MTX == 2 || na == 2) mfma_stage<NMAT, MTX, (MTX >= 2 ? 2 : 1)>(slot, xslot, trc, xrd, acc);
  else if (na == 3) mfma_stage<NMAT, MTX, (MTX >= 3 ? 3 : 1)>(slot, xslot, trc, xrd, acc);
  else mfma_stage<NMAT, MTX, (MTX >= 4 ? 4 : 1)>(slot, xslot, trc, xrd, acc);
}

// Stores the accumulators of the pass that just ended, by pair: up writes
// gate and up partial sums of slice ks, down the pair's output row.
template <int NMAT, bool UP>
__device__ __forceinline__ void epilogue(const Cursor &c, const Params &p, int wave, int lane,
                                         Acc<NMAT> &acc) {
  const int g = lane >> 4, j = lane & 15;
  const int T = min(kMaxTok, c.T - c.pass * kMaxTok);
  const int col = c.strip * kStripCols + 16 * wave + j;
  const int pbase = c.p0 + c.pass * kMaxTok;
  auto row = [&](int mat, int pr) { return UP ? size_t(c.ks * 2 + mat) * p.P + pr : size_t(pr); };
  if (T <= kDotMaxT) {
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
      for (int m = 0; m < kDotMaxT; ++m) {
        float v = acc.dot[mat][m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc.dot[mat][m] = v;
      }
    if (g == 0 && col < p.N) {
#pragma unroll
      for (int m = 0; m < kDotMaxT; ++m)
        if (m < T)
#pragma unroll
          for (int mat = 0; mat < NMAT; ++mat) p.out[row(mat, pbase + m) * p.N + col] = acc.dot[mat][m];
    }
    return;
  }
  if (col >= p.N) return;
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * t4 + 4 * g + i;
      if (m < T)
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) p.out[row(mat, pbase + m) * p.N + col] = acc.mf[mat][t4][i];
    }
}

template <int NMAT, int MTX, bool UP>
__global__ __launch_bounds__(kThreads, 1) void stream_kernel(
    Params p, const int32_t *__restrict__ n_active, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_token) {
  using S = Shape<NMAT, MTX>;
  constexpr int kS = S::kStages;
  constexpr int kD = kS - 1;  // stages in flight ahead of the one in use
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kS * S::kSlot + kMetaBytes];
  unsigned char *stages = lds;
  unsigned char *meta = lds + kS * S::kSlot;

  const int nact = n_active[0];
  const int total = offsets[nact];
  for (int i = threadIdx.x; i <= nact; i += kThreads) {
    reinterpret_cast<int16_t *>(meta + kMetaOff)[i] = int16_t(offsets[i]);
    if (i < nact) reinterpret_cast<int16_t *>(meta + kMetaAct)[i] = int16_t(active[i]);
  }
  for (int i = threadIdx.x; i < total; i += kThreads) meta[kMetaTok + i] = uint8_t(pair_token[i]);
  __syncthreads();

  const Stream<NMAT, MTX, UP> st(p, lds_addr(meta));
  Cursor cons;
  cons.per_expert = ((p.N + kStripCols - 1) / kStripCols) * p.slices;
  cons.n_items = nact * cons.per_expert;
  cons.item = blockIdx.x;
  st.decode(cons);
  if (!cons.valid) return;
  Cursor prod = cons;

  // Prologue: kD stages in flight. `issued` counts the stages issued so far.
  int issued = 0;
  for (int s = 0; s < kD; ++s) {
    if (!prod.valid) break;
    st.issue(prod, stages + s * S::kSlot);
    ++issued;
    st.advance(prod, gridDim.x);
  }

  Acc<NMAT> acc;
  clear(acc);
  const uint32_t base = lds_addr(stages);
  for (int s = 0; cons.valid; ++s) {
    // Stage s must have landed; the stages issued after it may stay in flight
    // (S::kCopies copies per wave each).
    const int newer = issued - s - 1;
    switch (newer < kD - 1 ? newer : kD - 1) {
      case 0: wait_barrier<0>(); break;
      case 1: wait_barrier<1 * S::kCopies>(); break;
      case 2: wait_barrier<2 * S::kCopies>(); break;
      case 3: wait_barrier<(kD - 1 >= 3 ? 3 : 0) * S::kCopies>(); break;
      case 4: wait_barrier<(kD - 1 >= 4 ? 4 : 0) * S::kCopies>(); break;
      default: wait_barrier<(kD - 1 >= 5 ? 5 : 0) * S::kCopies>(); break;
    }
    // Every wave is past stage s-1, so its slot takes stage s+kD.
    if (prod.valid) {
      st.issue(prod, stages + ((s + kD) % kS) * S::kSlot);
      ++issued;
      st.advance(prod, gridDim.x);
    }
    compute_stage<NMAT, MTX>(base + uint32_t((s % kS) * S::kSlot), st.trc, st.xrd, st.dotrd,
                             st.tp(cons), acc);
    if (cons.kst == cons.nst - 1) {
      epilogue<NMAT, UP>(cons, p, st.wave, st.lane, acc);
      clear(acc);
    }
    st.advance(cons, gridDim.x);
  }
}

// -------------------------------------------------------------------- h
// One thread per 4 consecutive columns of one pair. The thread of column 0
// also records the pair index of the pair's (token, slot), for the combine.
__global__ __launch_bounds__(kThreads) void h_kernel(const float *__restrict__ gpart, int nks,
                                                     int P, int I, int k,
                                                     const int32_t *__restrict__ n_active,
                                                     const int32_t *__restrict__ offsets,
                                                     const int32_t *__restrict__ pair_token,
                                                     const int32_t *__restrict__ pair_slot,
                                                     uint16_t *__restrict__ h,
                                                     int32_t *__restrict__ pair_of_slot) {
  const int total = offsets[n_active[0]];
  const int q4 = I / 4;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total * q4) return;
  const int pr = idx / q4;
  const int c = (idx - pr * q4) * 4;
  if (c == 0) pair_of_slot[pair_token[pr] * k + pair_slot[pr]] = pr;
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

// y[t] = sum over slots j in order of w[t,j] * part[pair of (t,j)] (empty
// slots skipped).
template <typename OutT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float *__restrict__ part,
                                                           const int32_t *__restrict__ pair_of_slot,
                                                           const int32_t *__restrict__ topk_ids,
                                                           const float *__restrict__ topk_w,
                                                           int B, int d, int k, OutT *__restrict__ y) {
  const int q4 = d / 4;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= B * q4) return;
  const int t = idx / q4;
  const int c = (idx - t * q4) * 4;
  float4 acc = make_float4(0, 0, 0, 0);
  for (int j = 0; j < k; ++j) {
    if (topk_ids[t * k + j] < 0) continue;
    const float w = topk_w[t * k + j];
    const float4 v = *reinterpret_cast<const float4 *>(part + size_t(pair_of_slot[t * k + j]) * d + c);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  store4<OutT>(y + size_t(t) * d + c, acc);
}

// ----------------------------------------------------------- float32 path
// One thread per (pair, column of I): h = SiLU(x G) * (x U), float32.
__global__ __launch_bounds__(kThreads) void up_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wg, const float *__restrict__ wu, int d,
    int I, int k, const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_token, const int32_t *__restrict__ pair_slot,
    const int32_t *__restrict__ topk_ids, float *__restrict__ h, int32_t *__restrict__ pair_of_slot) {
  const int total = offsets[n_active[0]];
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total * I) return;
  const int pr = idx / I, c = idx - pr * I;
  const int t = pair_token[pr];
  const int e = topk_ids[t * k + pair_slot[pr]];
  if (c == 0) pair_of_slot[t * k + pair_slot[pr]] = pr;
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

// One thread per (pair, column of d): part[pair] = h D, float32.
__global__ __launch_bounds__(kThreads) void down_f32_kernel(
    const float *__restrict__ h, const float *__restrict__ wd, int d, int I, int k,
    const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_token, const int32_t *__restrict__ pair_slot,
    const int32_t *__restrict__ topk_ids, float *__restrict__ part) {
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
  part[size_t(pr) * d + c] = acc;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

template <int NMAT, bool UP>
void launch_stream(int mtx, int grid, const Params &p, const moe_routing_t &r, hipStream_t s) {
  switch (mtx) {
    case 1:
      stream_kernel<NMAT, 1, UP><<<grid, kThreads, 0, s>>>(p, r.n_active, r.active_experts,
                                                         r.expert_offsets, r.pair_token);
      break;
    case 2:
      stream_kernel<NMAT, 2, UP><<<grid, kThreads, 0, s>>>(p, r.n_active, r.active_experts,
                                                         r.expert_offsets, r.pair_token);
      break;
    default:
      stream_kernel<NMAT, 4, UP><<<grid, kThreads, 0, s>>>(p, r.n_active, r.active_experts,
                                                         r.expert_offsets, r.pair_token);
      break;
  }
}

}  // namespace

hipError_t launch_expert_ffn(const void *x, const void *w_gate, const void *w_up,
                             const void *w_down, moe_dtype_t dt, int B, int d, int E, int I,
                             int k, const moe_routing_t &r, void *y, char *ws,
                             const Workspace &plan, hipStream_t s) {
  const int P = B * k;
  const int max_active = E < P ? E : P;
  float *part = reinterpret_cast<float *>(ws + plan.down_part);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + plan.pair_of_slot);
  if (dt == MOE_BF16) {
    float *gpart = reinterpret_cast<float *>(ws + plan.up_part);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + plan.h);
    const int cus = device_cus();
    // An expert has at most B tokens: A tiles of 16 * mtx rows cover them
    // (experts with more than 64 tokens take several passes).
    const int mtx = B <= 16 ? 1 : B <= 32 ? 2 : 4;

    Params up{};
    up.A = static_cast<const uint16_t *>(x);
    up.a_bytes = uint32_t(size_t(B) * d * 2);
    up.a_ld = d;
    up.W[0] = static_cast<const uint16_t *>(w_gate);
    up.W[1] = static_cast<const uint16_t *>(w_up);
    up.K = d;
    up.N = I;
    up.slices = plan.up_slices;
    up.slice_rows = plan.up_slice_rows;
    up.P = P;
    up.out = gpart;
    const int up_items = max_active * ceil_div(I, kStripCols) * plan.up_slices;
    launch_stream<2, true>(mtx, up_items < cus ? up_items : cus, up, r, s);

    h_kernel<<<ceil_div(P * (I / 4), kThreads), kThreads, 0, s>>>(
        gpart, plan.up_slices, P, I, k, r.n_active, r.expert_offsets, r.pair_token, r.pair_slot, h,
        pos);

    Params dn = up;
    dn.A = h;
    dn.a_bytes = uint32_t(size_t(P) * I * 2);
    dn.a_ld = I;
    dn.W[0] = static_cast<const uint16_t *>(w_down);
    dn.W[1] = nullptr;
    dn.K = I;
    dn.N = d;
    dn.slices = 1;
    dn.slice_rows = I;
    dn.out = part;
    const int down_items = max_active * ceil_div(d, kStripCols);
    launch_stream<1, false>(mtx, down_items < cus ? down_items : cus, dn, r, s);

    combine_kernel<uint16_t><<<ceil_div(B * (d / 4), kThreads), kThreads, 0, s>>>(
        part, pos, r.topk_ids, r.topk_w, B, d, k, static_cast<uint16_t *>(y));
  } else {
    float *h = reinterpret_cast<float *>(ws + plan.h);
    up_f32_kernel<<<ceil_div(P * I, kThreads), kThreads, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(w_gate),
        static_cast<const float *>(w_up), d, I, k, r.n_active, r.expert_offsets, r.pair_token,
        r.pair_slot, r.topk_ids, h, pos);
    down_f32_kernel<<<ceil_div(P * d, kThreads), kThreads, 0, s>>>(
        h, static_cast<const float *>(w_down), d, I, k, r.n_active, r.expert_offsets,
        r.pair_token, r.pair_slot, r.topk_ids, part);
    combine_kernel<float><<<ceil_div(B * (d / 4), kThreads), kThreads, 0, s>>>(
        part, pos, r.topk_ids, r.topk_w, B, d, k, static_cast<float *>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
