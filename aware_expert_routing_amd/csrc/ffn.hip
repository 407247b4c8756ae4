// Grouped SwiGLU expert FFN over the batch's active experts:
//   y[t] = sum_j w[t,j] * (SiLU(x_t G_e) * (x_t U_e)) D_e,  e = slot j's expert,
// reading only the weights of experts in the active list ("Lynx", Technical
// Summary 1: decode latency follows the number of distinct experts loaded;
// "Opportunistic Expert Activation", abstract: MoE latency is governed by the
// number of activated experts).
//
// bf16 path: one persistent kernel, one workgroup per CU.
//   * Work items: gate/up items (active expert x 64-column strip of I x slice
//     of d) come first, then down items (active expert x 128-column strip of
//     d x all of I); workgroup b takes items b, b+G, b+2G, ...
//   * Every item is a sequence of stages of kBK reduction rows; a stage holds
//     two weight tiles (G and U, or two adjacent 64-column tiles of D) and the
//     A tile of the same rows (x rows gathered by token, or h rows by pair).
//     Stages are copied HBM -> LDS with buffer_load ... lds (no registers
//     involved) into a ring of slots, several stages ahead of the one in use,
//     across item and phase boundaries.
//   * Each wave counts the copies it has issued and waits with s_waitcnt
//     vmcnt(n) for exactly the stage it needs, then one s_barrier.
//   * Weight rows are stored with their 16-byte chunks XOR-swizzled so that
//     the transposing LDS reads (ds_read_b64_tr_b16) that build MFMA B
//     fragments along the reduction dimension are bank-conflict free.
//   * An expert's tokens form the A operand: 16-row tiles of
//     v_mfma_f32_16x16x32_bf16, up to 64 tokens per pass.
//   * Gate/up slice partial sums go to the workspace; after a grid barrier
//     the grid forms h = SiLU(g) * u; after a second one the down items run.
//   * A down pass adds its tokens to per-(16-token group, strip) counters;
//     the workgroup that completes a group's count forms y over that strip
//     for the group's tokens, adding the slots in order (no float atomics:
//     results are reproducible).
// float32 path (small layers): plain dot products, 16 row groups per column.
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
constexpr int kMaxPairs = kMaxB * kMaxK;
constexpr int kSliceCost = 8;  // stages' worth of time the sliced gate/up path adds (measured)
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, gfx9 data format
constexpr int kLdsBytes = 160 * 1024;
static_assert(kStripCols == 64 && kBK == 128, "tile constants");

// Routing lists staged in LDS once per workgroup (the loop reads them with
// the inline-assembly helpers below). Every field is aligned to its element
// size (LDS atomics need natural alignment) and the area to 16 bytes.
constexpr int kMetaLast = 0;                            // int32 token groups whose strip this pass completes
constexpr int kMetaNLast = kMetaLast + 4 * kMaxTok;     // int32 their number
constexpr int kMetaFill = kMetaNLast + 16;              // uint32 filled slots of each token
constexpr int kMetaRow = kMetaFill + 4 * kMaxB;         // int16 token slot t*k+j of each pair
constexpr int kMetaAct = kMetaRow + 2 * kMaxPairs;      // int16 active expert list
constexpr int kMetaOff = kMetaAct + 2 * kMaxE;          // int16 CSR offsets
constexpr int kMetaGFill = kMetaOff + 2 * (kMaxE + 1) + 2;  // uint32 filled slots of each token group
constexpr int kMetaTok = kMetaGFill + 4 * kTokGroups;   // uint8 token of each pair
constexpr int kMetaBytes = (kMetaTok + kMaxPairs + 15) / 16 * 16;
static_assert(kMetaNLast % 4 == 0 && kMetaFill % 4 == 0 && kMetaRow % 2 == 0 && kMetaAct % 2 == 0 &&
                  kMetaOff % 2 == 0 && kMetaGFill % 4 == 0,
              "meta field alignment");

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

// XOR applied to the 16-byte chunk index of weight row r of a stage (an even
// value, so chunk pairs 2c, 2c+1 stay together). The 16 lanes of group g of a
// transposing read take rows kk + 8g + 4h + {0..3}, 32 bytes (one chunk pair)
// each; the XOR differs between those four rows, so the group covers all 32
// banks once. It does not depend on kk (a multiple of 32), so a lane's read
// offsets are constants.
__device__ __forceinline__ int swz_w(int r) { return ((r ^ (r >> 2)) & 3) << 1; }
// Chunk XOR of A-tile row m (rows of 64 bytes = 4 chunks): the 8 lanes
// (rows j..j+7, one logical chunk) that a 16-byte read serves together hit 8
// distinct 4-bank groups.
__device__ __forceinline__ int swz_x(int m) { return (m >> 1) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kRsrcWord3);
}

// Cache-policy bits of a memory instruction: SC1 makes it coherent at device
// scope (across XCDs), which data exchanged between workgroups of one kernel
// needs.
constexpr int kPolicyDevice = 16;
// NT marks a copy as streaming (read once): the expert weights are copied
// with it, which was measured to shorten every stage of the kernel (the
// weights then do not displace reused lines in the caches).
constexpr int kPolicyStream = 2;

// Copies 16 bytes per lane from buffer offset voff + soff into LDS at
// dst + 16*lane. Offsets at or past the end of the buffer read as zero.
template <int POLICY = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff,
                                      uint32_t soff) {
  // A C-style cast is the way to move a generic pointer into the LDS address space.
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst), 16, int(voff), int(soff), 0, POLICY);
}

// Device-scope stores and loads of data that other workgroups of the same
// kernel read or wrote (partial sums, h, down rows, the slot map). They reach
// or come from the device-coherent level directly, so the grid barrier needs
// no cache write-back or invalidation.
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at byte offset `off` of buffer r, device scope.
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const f32x4_t v = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kPolicyDevice));
  return make_float4(v[0], v[1], v[2], v[3]);
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

// Grid-barrier words in the workspace, each on its own 128-byte line: the
// arrival count (counts every arrival of the launch, zero at launch start and
// end), the release word (counts completed barriers, never reset) and the
// error flag. Arrivals and polls touch different lines, so polling does not
// slow the arrivals' atomics.
constexpr int kSyncCount = 0;
constexpr int kSyncRelease = 32;
constexpr int kSyncErr = 64;
constexpr uint32_t kSpinLimit = 1u << 20;

// The release word as the launch found it. Every workgroup reads it before
// its first arrival and no barrier completes before every workgroup has
// arrived, so all of them read the same value.
__device__ __forceinline__ uint32_t release_base(const uint32_t *sync) {
  return __hip_atomic_load(const_cast<uint32_t *>(sync) + kSyncRelease, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier `index` (1, 2, ... within a launch) of all workgroups of the grid
// (resident together: one per CU at most); one wave of each workgroup takes
// part (its lanes wait for lane 0). An arrival is one atomic add whose old
// value tells whether it completes the barrier; the last arriver stores
// base + index into the release word, the others poll that word. The final
// barrier's last arriver puts the count back to zero for the next launch
// (nothing else touches it in this launch). Every store that another
// workgroup reads after the barrier is a device-scope store made before the
// arrival by a wave whose stores have completed (s_waitcnt vmcnt(0)), and
// those reads are device-scope loads, so no cache maintenance is needed. A
// wait that does not end within kSpinLimit polls sets the error word and
// returns, so the kernel always terminates.
__device__ __forceinline__ void grid_barrier_wave(uint32_t *sync, uint32_t base, uint32_t index,
                                                  bool final_barrier) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(sync + kSyncCount, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = base + index;
    if (before == index * gridDim.x - 1) {
      if (final_barrier) __hip_atomic_store(sync + kSyncCount, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + kSyncRelease, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      for (uint32_t n = 0;
           __hip_atomic_load(sync + kSyncRelease, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target;
           ++n) {
        if (n >= kSpinLimit) {
          __hip_atomic_store(sync + kSyncErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

struct Params {
  const uint16_t *x;          // [B, d]
  const uint16_t *W[3];       // G, U: [E, d, I]; D: [E, I, d]
  int B, d, E, I, k;
  int slices, slice_rows;     // gate/up reduction slices over d (1: whole of d, h formed in the epilogue)
  int P;                      // B * k
  float *gpart;               // [slices][2][P][I] gate/up partial sums by pair
  uint16_t *h;                // [P][I] SiLU(g) * u by pair
  float *part;                // [P][d] down-projection rows by token slot t*k+j
  uint16_t *y;                // [B][d]
  const int32_t *ids;         // [B][k]
  const float *w;             // [B][k]
  const int32_t *pair_token;  // [P]
  const int32_t *pair_slot;   // [P]
  uint32_t *sync;             // grid-barrier words
  uint32_t *grp_cnt;          // per (strip, token group): slots counted, one 128-byte line each
  int n_dstrips;              // 128-column strips of d
};

// By active-expert count: gate/up stages of kBK rows per d slice (all of d
// for whole tiles). A kernel argument of its own, never written, so that the
// kernel reads the entry it needs from the argument segment.
struct UpPlan {
  uint32_t e2[(kMaxE + 2) / 2];  // entry n in half n % 2 of word n / 2: stages per slice | slices << 8
};

// A position in a workgroup's stage sequence. The workgroup's items are
// b, b+G, b+2G, ... of one list: gate/up items first (expert, 64-column strip
// of I, slice of d), then down items (expert, 128-column strip of d, all of
// I). Every stage holds two weight tiles (G and U, or two adjacent 64-column
// tiles of D) and the A tile of the same reduction rows (x rows gathered by
// token, or h rows by pair). All fields are wave-uniform.
struct Cursor {
  int item, n_items, n_up, per_up, per_dn;
  int e, p0, T, strip, ks, row0, nrows, nst, npass, pass, kst;
  bool valid, up;
};

template <int MTX>
struct Stream {
  using S = Shape<2, MTX>;
  const Params &p;
  uint32_t meta;            // LDS address of the routing lists
  int wave, lane, g, j;
  uint32_t wv_up[4];        // weight copy offsets within a stage (row stride I)
  uint32_t wv_dn[4];        // the same for D (row stride d)
  uint32_t trc[2];          // transposing-read offsets within a weight tile
  uint32_t xrd;             // A-fragment read offset within a k-step sub-tile

  __device__ __forceinline__ Stream(const Params &pp, uint32_t meta_addr) : p(pp), meta(meta_addr) {
    wave = wave_id();
    lane = threadIdx.x & 63;
    g = lane >> 4;
    j = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = 8 * (wave + 4 * h) + (lane >> 3);
      const int lc = (lane & 7) ^ swz_w(r);
      wv_up[h] = uint32_t(r) * uint32_t(p.I) * 2u + uint32_t(lc) * 16u;
      wv_dn[h] = uint32_t(r) * uint32_t(p.d) * 2u + uint32_t(lc) * 16u;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R = 8 * g + 4 * h + (j >> 2);
      const int c = 2 * wave + ((j & 3) >> 1);
      trc[h] = uint32_t(R * kRowBytes + ((c ^ swz_w(R)) << 4) + ((j & 1) << 3));
    }
    xrd = uint32_t(j * 64 + ((g ^ swz_x(j)) << 4));
  }

  __device__ __forceinline__ void decode(Cursor &c) const {
    c.valid = c.item < c.n_items;
    if (!c.valid) return;
    c.up = c.item < c.n_up;
    int a;
    if (c.up) {
      a = c.item / c.per_up;
      const int rem = c.item - a * c.per_up;
      c.strip = rem / p.slices;
      c.ks = rem - c.strip * p.slices;
      c.row0 = c.ks * p.slice_rows;
      c.nrows = min(p.slice_rows, p.d - c.row0);
    } else {
      const int jd = c.item - c.n_up;
      a = jd / c.per_dn;
      c.strip = jd - a * c.per_dn;
      c.ks = 0;
      c.row0 = 0;
      c.nrows = p.I;
    }
    c.e = __builtin_amdgcn_readfirstlane(lds_i16(meta + kMetaAct + 2 * a));
    c.p0 = __builtin_amdgcn_readfirstlane(lds_i16(meta + kMetaOff + 2 * a));
    c.T = __builtin_amdgcn_readfirstlane(lds_i16(meta + kMetaOff + 2 * a + 2)) - c.p0;
    c.nst = (c.nrows + kBK - 1) / kBK;
    c.npass = (c.T + kMaxTok - 1) / kMaxTok;
    c.pass = 0;
    c.kst = 0;
  }
  __device__ __forceinline__ void advance(Cursor &c) const {
    if (++c.kst < c.nst) return;
    c.kst = 0;
    if (++c.pass < c.npass) return;
    c.item += gridDim.x;
    decode(c);
  }
  __device__ __forceinline__ static int tp(const Cursor &c) { return min(kMaxTok, c.T - c.pass * kMaxTok); }

  // Byte offset of the A row this lane copies for its copy h (MTX copies per
  // wave, one 16-row tile each, all at k-step `wave` of the stage).
  __device__ __forceinline__ uint32_t xvoff(const Cursor &c, int h) const {
    const int m = 16 * h + (lane >> 2);
    const int T = tp(c);
    const int pr = c.p0 + c.pass * kMaxTok + (m < T ? m : T - 1);
    const int lc = (lane & 3) ^ swz_x(m);
    const uint32_t kofs = uint32_t(wave * 32 + lc * 8);
    if (c.up) return (uint32_t(lds_u8(meta + kMetaTok + pr)) * uint32_t(p.d) + kofs) * 2u;
    return (uint32_t(pr) * uint32_t(p.I) + kofs) * 2u;
  }

  // The A-tile copies of stage c (MTX per wave): x rows by token for gate/up,
  // h rows by pair for down (device scope: other workgroups wrote h).
  __device__ __forceinline__ void issue_a(const Cursor &c, unsigned char *slot) const {
    unsigned char *dst = slot + 2 * kWTile + wave * S::kXSub;
    const uint32_t xsoff = uint32_t(c.row0 + c.kst * kBK) * 2u;
    if (c.up) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.x, uint32_t(p.B) * uint32_t(p.d) * 2u);
#pragma unroll
      for (int h = 0; h < MTX; ++h) dma16(ra, dst + h * 1024, xvoff(c, h), xsoff);
    } else {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.h, uint32_t(p.P) * uint32_t(p.I) * 2u);
#pragma unroll
      for (int h = 0; h < MTX; ++h) dma16<kPolicyDevice>(ra, dst + h * 1024, xvoff(c, h), xsoff);
    }
  }

  // The weight copies of down stage c that wave `vw` normally issues (4 per
  // tile), issued by this wave: used while wave 0 is busy at the grid barriers.
  __device__ __forceinline__ void issue_dn_weights_as(const Cursor &c, unsigned char *slot, int vw) const {
    const size_t base = size_t(c.e) * p.I * p.d;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p.W[2] + base, uint32_t(p.I) * uint32_t(p.d) * 2u);
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      const uint32_t soff = (uint32_t(c.kst * kBK) * uint32_t(p.d) +
                             uint32_t((2 * c.strip + mat) * kStripCols)) * 2u;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int rr = 8 * (vw + 4 * h) + (lane >> 3);
        const uint32_t voff = uint32_t(rr) * uint32_t(p.d) * 2u + uint32_t((lane & 7) ^ swz_w(rr)) * 16u;
        dma16<kPolicyStream>(r, slot + mat * kWTile + (vw + 4 * h) * 1024, voff, soff);
      }
    }
  }

  // Issues half of this wave's copies of stage c into `slot`: half 0 the
  // first weight tile and the A tile, half 1 the second weight tile
  // (S::kCopies per wave in all).
  __device__ __forceinline__ void issue_half(const Cursor &c, unsigned char *slot, int half) const {
    if (c.up) {
      const size_t base = (size_t(c.e) * p.d + c.row0) * p.I;
      const uint32_t wbytes = uint32_t(c.nrows) * uint32_t(p.I) * 2u;
      const uint32_t soff =
          (uint32_t(c.kst * kBK) * uint32_t(p.I) + uint32_t(c.strip * kStripCols)) * 2u;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p.W[half] + base, wbytes);
#pragma unroll
      for (int h = 0; h < 4; ++h) dma16<kPolicyStream>(r, slot + half * kWTile + (wave + 4 * h) * 1024, wv_up[h], soff);
    } else {
      const size_t base = size_t(c.e) * p.I * p.d;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p.W[2] + base, uint32_t(p.I) * uint32_t(p.d) * 2u);
      const uint32_t soff = (uint32_t(c.kst * kBK) * uint32_t(p.d) +
                             uint32_t((2 * c.strip + half) * kStripCols)) * 2u;
#pragma unroll
      for (int h = 0; h < 4; ++h) dma16<kPolicyStream>(r, slot + half * kWTile + (wave + 4 * h) * 1024, wv_dn[h], soff);
    }
    if (half == 0) issue_a(c, slot);
  }
  // Issues every copy of stage c into `slot`.
  __device__ __forceinline__ void issue(const Cursor &c, unsigned char *slot) const {
    issue_half(c, slot, 0);
    issue_half(c, slot, 1);
  }
};

struct Acc {
  f32x4_t mf[2][4];  // rows 4*(lane/16)+i of tile mt, column 16*wave + lane%16
};

__device__ __forceinline__ void clear(Acc &acc) {
#pragma unroll
  for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc.mf[mat][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Operand fragments of k-steps 2*KP and 2*KP+1 of a stage, read from LDS by
// one inline-assembly block that waits once, so that the reads of two
// k-steps overlap. Per k-step ks:
//   B fragments (column 16*wave + j, rows 32ks + 8g .. +7 of both weight
//   tiles): four transposing reads at the lane's offsets b0 and b1 (rows
//   8g + 4h + j/4 of the k-step), in tile 0 and in tile 1 (kWTile further);
//   the read gives lane j of a 16-lane group element j of the four rows its
//   group's lanes point at (lane 4r+q points at row r, columns 4q..4q+3);
//   A fragments: NA reads of 16 bytes at xa[mt] + ks * XS (row tile mt).
#define MOE_TR_PAIR(J)                                                   \
  "ds_read_b64_tr_b16 %[t" #J "0], %[B0] offset:%[ob" #J "]\n\t"         \
  "ds_read_b64_tr_b16 %[t" #J "1], %[B1] offset:%[ob" #J "]\n\t"         \
  "ds_read_b64_tr_b16 %[t" #J "2], %[B0] offset:%[ow" #J "]\n\t"         \
  "ds_read_b64_tr_b16 %[t" #J "3], %[B1] offset:%[ow" #J "]\n\t"
#define MOE_TR_OUTS                                                            \
  [t00] "=&v"(t[0][0]), [t01] "=&v"(t[0][1]), [t02] "=&v"(t[0][2]), [t03] "=&v"(t[0][3]), \
  [t10] "=&v"(t[1][0]), [t11] "=&v"(t[1][1]), [t12] "=&v"(t[1][2]), [t13] "=&v"(t[1][3])
#define MOE_TR_INS(KP)                                                          \
  [B0] "v"(b0), [B1] "v"(b1), [ob0] "i"((2 * KP) * 32 * kRowBytes),             \
  [ob1] "i"((2 * KP + 1) * 32 * kRowBytes), [ow0] "i"((2 * KP) * 32 * kRowBytes + kWTile), \
  [ow1] "i"((2 * KP + 1) * 32 * kRowBytes + kWTile), [oa0] "i"((2 * KP) * XS), [oa1] "i"((2 * KP + 1) * XS)

template <int NA, int KP, int XS>
struct PairFrags;

template <int KP, int XS>
struct PairFrags<1, KP, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][4], bf16x8_t (&a)[2][4]) {
    asm volatile(MOE_TR_PAIR(0) MOE_TR_PAIR(1)
                 "ds_read_b128 %[a00], %[X0] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a10], %[X0] offset:%[oa1]\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MOE_TR_OUTS, [a00] "=&v"(a[0][0]), [a10] "=&v"(a[1][0])
                 : MOE_TR_INS(KP), [X0] "v"(xa[0]));
  }
};
template <int KP, int XS>
struct PairFrags<2, KP, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][4], bf16x8_t (&a)[2][4]) {
    asm volatile(MOE_TR_PAIR(0) MOE_TR_PAIR(1)
                 "ds_read_b128 %[a00], %[X0] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a01], %[X1] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a10], %[X0] offset:%[oa1]\n\t"
                 "ds_read_b128 %[a11], %[X1] offset:%[oa1]\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MOE_TR_OUTS, [a00] "=&v"(a[0][0]), [a01] "=&v"(a[0][1]), [a10] "=&v"(a[1][0]),
                   [a11] "=&v"(a[1][1])
                 : MOE_TR_INS(KP), [X0] "v"(xa[0]), [X1] "v"(xa[1]));
  }
};
template <int KP, int XS>
struct PairFrags<3, KP, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][4], bf16x8_t (&a)[2][4]) {
    asm volatile(MOE_TR_PAIR(0) MOE_TR_PAIR(1)
                 "ds_read_b128 %[a00], %[X0] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a01], %[X1] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a02], %[X2] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a10], %[X0] offset:%[oa1]\n\t"
                 "ds_read_b128 %[a11], %[X1] offset:%[oa1]\n\t"
                 "ds_read_b128 %[a12], %[X2] offset:%[oa1]\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MOE_TR_OUTS, [a00] "=&v"(a[0][0]), [a01] "=&v"(a[0][1]), [a02] "=&v"(a[0][2]),
                   [a10] "=&v"(a[1][0]), [a11] "=&v"(a[1][1]), [a12] "=&v"(a[1][2])
                 : MOE_TR_INS(KP), [X0] "v"(xa[0]), [X1] "v"(xa[1]), [X2] "v"(xa[2]));
  }
};
template <int KP, int XS>
struct PairFrags<4, KP, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][4], bf16x8_t (&a)[2][4]) {
    asm volatile(MOE_TR_PAIR(0) MOE_TR_PAIR(1)
                 "ds_read_b128 %[a00], %[X0] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a01], %[X1] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a02], %[X2] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a03], %[X3] offset:%[oa0]\n\t"
                 "ds_read_b128 %[a10], %[X0] offset:%[oa1]\n\t"
                 "ds_read_b128 %[a11], %[X1] offset:%[oa1]\n\t"
                 "ds_read_b128 %[a12], %[X2] offset:%[oa1]\n\t"
                 "ds_read_b128 %[a13], %[X3] offset:%[oa1]\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : MOE_TR_OUTS, [a00] "=&v"(a[0][0]), [a01] "=&v"(a[0][1]), [a02] "=&v"(a[0][2]),
                   [a03] "=&v"(a[0][3]), [a10] "=&v"(a[1][0]), [a11] "=&v"(a[1][1]),
                   [a12] "=&v"(a[1][2]), [a13] "=&v"(a[1][3])
                 : MOE_TR_INS(KP), [X0] "v"(xa[0]), [X1] "v"(xa[1]), [X2] "v"(xa[2]), [X3] "v"(xa[3]));
  }
};
#undef MOE_TR_PAIR
#undef MOE_TR_OUTS
#undef MOE_TR_INS

// MFMA work of one stage in two pairs of k-steps; hook(kp) runs before pair
// kp (the loop issues half of a later stage's copies there, so that the
// copies enter the memory pipeline while this stage computes).
template <int MTX, int NA, class Hook>
__device__ __forceinline__ void mfma_stage(uint32_t slot, uint32_t xslot, const uint32_t (&trc)[2],
                                           uint32_t xrd, Acc &acc, const Hook &hook) {
  constexpr int XS = Shape<2, MTX>::kXSub;
  static_assert(kKSteps == 4, "two pairs of k-steps per stage");
  const uint32_t b0 = slot + trc[0], b1 = slot + trc[1];
  uint32_t xa[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) xa[mt] = xslot + uint32_t(mt * 1024) + xrd;
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    hook(kp);
    long t[2][4];
    bf16x8_t a[2][4];
    if (kp == 0) PairFrags<NA, 0, XS>::read(b0, b1, xa, t, a);
    else PairFrags<NA, 1, XS>::read(b0, b1, xa, t, a);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bf16x8_t b[2];
      __builtin_memcpy(&b[0], &t[q][0], 8);
      __builtin_memcpy(reinterpret_cast<char *>(&b[0]) + 8, &t[q][1], 8);
      __builtin_memcpy(&b[1], &t[q][2], 8);
      __builtin_memcpy(reinterpret_cast<char *>(&b[1]) + 8, &t[q][3], 8);
#pragma unroll
      for (int mt = 0; mt < NA; ++mt)
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
          acc.mf[mat][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q][mt], b[mat], acc.mf[mat][mt], 0, 0, 0);
    }
  }
}

template <int MTX, class Hook>
__device__ __forceinline__ void compute_stage(uint32_t slot, const uint32_t (&trc)[2], uint32_t xrd,
                                              int T, Acc &acc, const Hook &hook) {
  const uint32_t xslot = slot + 2 * kWTile;
  const int na = (T + 15) >> 4;
  if (MTX == 1 || na == 1) mfma_stage<MTX, 1>(slot, xslot, trc, xrd, acc, hook);
  else if (MTX == 2 || na == 2) mfma_stage<MTX, (MTX >= 2 ? 2 : 1)>(slot, xslot, trc, xrd, acc, hook);
  else if (na == 3) mfma_stage<MTX, (MTX >= 3 ? 3 : 1)>(slot, xslot, trc, xrd, acc, hook);
  else mfma_stage<MTX, (MTX >= 4 ? 4 : 1)>(slot, xslot, trc, xrd, acc, hook);
}

// Stores the accumulators of the pass that just ended: the gate and up partial
// sums of slice ks by pair, or two 64-column tiles of the down projection by
// token slot.
// A pass has at most 16 * MTX tokens.
template <int MTX>
__device__ __forceinline__ void epilogue(const Cursor &c, const Params &p, uint32_t meta, int wave,
                                         int lane, Acc &acc) {
  const int g = lane >> 4, j = lane & 15;
  const int T = min(kMaxTok, c.T - c.pass * kMaxTok);
  const int pbase = c.p0 + c.pass * kMaxTok;
  if (c.up && p.slices == 1) {
    // The whole reduction is in the accumulators: h = SiLU(g) * u by pair.
    const int col = c.strip * kStripCols + 16 * wave + j;
    if (col < p.I) {
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.h, uint32_t(p.P) * uint32_t(p.I) * 2u);
#pragma unroll
      for (int t4 = 0; t4 < MTX; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * t4 + 4 * g + i;
          if (m < T) {
            const uint16_t hv = f32_to_bf16(silu(acc.mf[0][t4][i]) * acc.mf[1][t4][i]);
            __builtin_amdgcn_raw_buffer_store_b16(hv, rh, int((uint32_t(pbase + m) * uint32_t(p.I) + uint32_t(col)) * 2u),
                                                  0, kPolicyDevice);
          }
        }
    }
    return;
  }
  float *dst0, *dst1;
  int col0, col1, ld;
  if (c.up) {
    ld = p.I;
    col0 = col1 = c.strip * kStripCols + 16 * wave + j;
    dst0 = p.gpart + size_t(c.ks * 2) * p.P * p.I;
    dst1 = dst0 + size_t(p.P) * p.I;
  } else {
    ld = p.d;
    col0 = 2 * c.strip * kStripCols + 16 * wave + j;
    col1 = col0 + kStripCols;
    dst0 = dst1 = p.part;
  }
  const bool ok0 = col0 < ld, ok1 = col1 < ld;
#pragma unroll
  for (int t4 = 0; t4 < MTX; ++t4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * t4 + 4 * g + i;
      if (m < T) {
        const size_t row = size_t(c.up ? pbase + m : lds_i16(meta + kMetaRow + 2 * (pbase + m))) * ld;
        if (ok0) st_dev(dst0 + row + col0, acc.mf[0][t4][i]);
        if (ok1) st_dev(dst1 + row + col1, acc.mf[1][t4][i]);
      }
    }
}

// h = SiLU(g) * u from the slice partial sums, spread over waves 0 and 1 of
// every workgroup (threads 0..127). All loads of a lane are issued before the
// first is used; the stores have completed when it returns.
__device__ __forceinline__ void h_phase_waves01(const Params &p, int total) {
  const int q4 = p.I / 4;
  const int n = total * q4;
  const uint32_t blk = uint32_t(p.P) * uint32_t(p.I) * 4u;  // bytes of one [P][I] block
  for (int idx = blockIdx.x * 128 + threadIdx.x; idx < n; idx += gridDim.x * 128) {
    const int pr = idx / q4;
    const int c = (idx - pr * q4) * 4;
    const uint32_t off = (uint32_t(pr) * uint32_t(p.I) + uint32_t(c)) * 4u;
    float4 gv[kUpMaxSlices], uv[kUpMaxSlices];
#pragma unroll
    for (int s = 0; s < kUpMaxSlices; ++s) {
      if (s < p.slices) {
        gv[s] = ld_dev4(make_rsrc(p.gpart + size_t(s * 2 + 0) * p.P * p.I, blk), off);
        uv[s] = ld_dev4(make_rsrc(p.gpart + size_t(s * 2 + 1) * p.P * p.I, blk), off);
      }
    }
    float4 g = make_float4(0, 0, 0, 0), u = make_float4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < kUpMaxSlices; ++s) {
      if (s < p.slices) {
        g.x += gv[s].x; g.y += gv[s].y; g.z += gv[s].z; g.w += gv[s].w;
        u.x += uv[s].x; u.y += uv[s].y; u.z += uv[s].z; u.w += uv[s].w;
      }
    }
    const uint64_t o = uint64_t(f32_to_bf16(silu(g.x) * u.x)) |
                       (uint64_t(f32_to_bf16(silu(g.y) * u.y)) << 16) |
                       (uint64_t(f32_to_bf16(silu(g.z) * u.z)) << 32) |
                       (uint64_t(f32_to_bf16(silu(g.w) * u.w)) << 48);
    st_dev(reinterpret_cast<uint64_t *>(p.h + size_t(pr) * p.I + c), o);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// s_barrier without the wait for outstanding memory operations that
// __syncthreads adds: copies in flight stay in flight.
__device__ __forceinline__ void barrier_no_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Counter of (token group grp, down strip) on a 128-byte line of its own.
__device__ __forceinline__ uint32_t *group_counter(const Params &p, int grp, int strip) {
  return p.grp_cnt + (size_t(strip) * kTokGroups + grp) * kCntStride;
}

// y over 128-column strip `strip` for the tokens of group grp: thread i takes
// token 16*grp + i/16 and columns 8*(i%16) .. +7 of the strip, adding
// w[t,j] * part[t*k+j] in slot order (empty slots skipped). Slots are taken
// eight at a time with every load of a round issued before the first use.
static_assert(kThreads == kTokGroup * (2 * kStripCols / 8), "one thread per token and 8 columns");
__device__ __forceinline__ void combine_group(const Params &p, int grp, int strip) {
  const int t = grp * kTokGroup + (threadIdx.x >> 4);
  const int col = strip * 2 * kStripCols + (threadIdx.x & 15) * 8;
  if (t >= p.B || col >= p.d) return;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part, uint32_t(p.P) * uint32_t(p.d) * 4u);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < p.k; j0 += 8) {
    int id[8];
    float w[8];
    float4 v[8][2];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;
      if (j < p.k) {
        const int slot = t * p.k + j;
        id[jj] = p.ids[slot];
        w[jj] = p.w[slot];
        const uint32_t off = (uint32_t(slot) * uint32_t(p.d) + uint32_t(col)) * 4u;
        v[jj][0] = ld_dev4(rp, off);
        v[jj][1] = ld_dev4(rp, off + 16u);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < p.k && id[jj] >= 0) {
        acc[0] = fmaf(w[jj], v[jj][0].x, acc[0]);
        acc[1] = fmaf(w[jj], v[jj][0].y, acc[1]);
        acc[2] = fmaf(w[jj], v[jj][0].z, acc[2]);
        acc[3] = fmaf(w[jj], v[jj][0].w, acc[3]);
        acc[4] = fmaf(w[jj], v[jj][1].x, acc[4]);
        acc[5] = fmaf(w[jj], v[jj][1].y, acc[5]);
        acc[6] = fmaf(w[jj], v[jj][1].z, acc[6]);
        acc[7] = fmaf(w[jj], v[jj][1].w, acc[7]);
      }
    }
  }
  uint4 o;
  o.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
  o.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
  o.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
  o.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
  *reinterpret_cast<uint4 *>(p.y + size_t(t) * p.d + col) = o;
}

// End of a down pass (its rows stored by every wave). The pass adds, for
// each 16-token group it has tokens of, their number to the group's counter
// for the strip (one atomic per group, not per token: the atomics of one
// counter are served in turn). The workgroup that brings a counter to the
// group's number of filled slots forms y over the strip for the whole group
// (combine_group) and resets the counter. A count is taken only after this
// workgroup's stores have completed, so the last one finds every row of the
// group in place.
__device__ __forceinline__ void finish_down(const Cursor &c, const Params &p, unsigned char *meta,
                                            int wave, int lane) {
  const int T = min(kMaxTok, c.T - c.pass * kMaxTok);
  const int pbase = c.p0 + c.pass * kMaxTok;
  int32_t *last = reinterpret_cast<int32_t *>(meta + kMetaLast);
  int32_t *n_last = reinterpret_cast<int32_t *>(meta + kMetaNLast);
  const uint32_t *gfill = reinterpret_cast<const uint32_t *>(meta + kMetaGFill);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave == 0) {
    // The first lane of each run of lanes in one group adds the run's
    // length (an expert's tokens ascend, so a group is one run).
    const int grp = lane < T ? int(meta[kMetaTok + pbase + lane]) / kTokGroup : -1;
    const int prev = __shfl_up(grp, 1);
    const bool first = lane < T && (lane == 0 || prev != grp);
    const unsigned long long fb = __ballot(first);
    bool mine = false;
    if (first) {
      const unsigned long long above = lane == 63 ? 0ull : (fb >> (lane + 1));
      const int run = above ? __builtin_ctzll(above) + 1 : T - lane;
      const uint32_t before = __hip_atomic_fetch_add(group_counter(p, grp, c.strip), uint32_t(run),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mine = before + uint32_t(run) == gfill[grp];
    }
    const unsigned long long b = __ballot(mine);
    if (mine) last[__builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(b), 0))] = grp;
    if (lane == 0) *n_last = __popcll(b);
  }
  __syncthreads();
  const int n = *n_last;
  for (int q = 0; q < n; ++q) {
    const int grp = last[q];
    combine_group(p, grp, c.strip);
    if (threadIdx.x == 0)
      __hip_atomic_store(group_counter(p, grp, c.strip), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// y over the strips of token groups that have no filled slot at all (no
// down pass counts them): zero, written by workgroups b, b+G, ... of the
// (group, strip) units. Such groups only come from caller-made routings.
__device__ __forceinline__ void zero_empty_groups(const Params &p, const unsigned char *meta) {
  const uint32_t *gfill = reinterpret_cast<const uint32_t *>(meta + kMetaGFill);
  const int ngroups = (p.B + kTokGroup - 1) / kTokGroup;
  for (int u = blockIdx.x; u < ngroups * p.n_dstrips; u += gridDim.x) {
    const int grp = u / p.n_dstrips, strip = u - grp * p.n_dstrips;
    if (gfill[grp] != 0) continue;
    const int t = grp * kTokGroup + (threadIdx.x >> 4);
    const int col = strip * 2 * kStripCols + (threadIdx.x & 15) * 8;
    if (t < p.B && col < p.d) *reinterpret_cast<uint4 *>(p.y + size_t(t) * p.d + col) = make_uint4(0, 0, 0, 0);
  }
}

// The change from gate/up to down in a workgroup: every gate/up stage of it
// has been consumed and no down stage issued (the producer stops at the first
// one); `first` is the next stage index. Wave 0 meets the grid at the first
// barrier (gate/up partial sums complete); waves 0 and 1 then form this
// workgroup's share of h, and wave 0 meets the grid again (h complete).
// Meanwhile waves 2 and 3 copy the weights of the next kD down stages, all
// four shares, so those copies overlap the barriers without delaying the
// waits of waves 0 and 1 (vmcnt completes in order). Then every wave copies
// its h rows of those stages and waits for all of them.
template <int MTX>
__device__ __forceinline__ void change_to_down(const Params &p, const Stream<MTX> &st, Cursor &prod,
                                               int &issued, int first, unsigned char *stages,
                                               int total, uint32_t rel_base) {
  using S = Shape<2, MTX>;
  constexpr int kS = S::kStages;
  constexpr int kD = kS - 1;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's gate/up stores
  __syncthreads();
  const bool sliced = p.slices > 1;  // else the gate/up epilogues formed h
  if (st.wave == 0) {
    if (sliced) grid_barrier_wave(p.sync, rel_base, 1, false);
    else grid_barrier_wave(p.sync, rel_base, 1, true);
  } else if (st.wave >= 2) {
    Cursor q = prod;
    for (int n = 0; n < kD && q.valid; ++n) {
      unsigned char *slot = stages + ((first + n) % kS) * S::kSlot;
      st.issue_dn_weights_as(q, slot, st.wave - 2);
      st.issue_dn_weights_as(q, slot, st.wave);
      st.advance(q);
    }
  }
  barrier_no_wait();
  if (sliced) {
    if (st.wave < 2) h_phase_waves01(p, total);
    barrier_no_wait();
    if (st.wave == 0) grid_barrier_wave(p.sync, rel_base, 2, true);
    barrier_no_wait();
  }
  for (int n = 0; n < kD && prod.valid; ++n) {
    st.issue_a(prod, stages + ((first + n) % kS) * S::kSlot);
    st.advance(prod);
    ++issued;
  }
  wait_barrier<0>();
}

// The whole bf16 expert FFN in one persistent kernel (one workgroup per CU,
// all resident together):
//   1. gate/up items stream G and U and store slice partial sums;
//   2. grid barrier; h = SiLU(g) * u over the grid; grid barrier
//      (change_to_down);
//   3. down items stream D with h as the A operand and store rows by token
//      slot; each token's strip of y is formed by the workgroup that
//      completes it (finish_down).
// The first down stages' weights are in flight while the workgroup waits at
// the grid barriers; their A tiles are copied once h is complete.
template <int MTX>
__global__ __launch_bounds__(kThreads, 1) void ffn_kernel(Params p, const UpPlan up,
                                                          const int32_t *__restrict__ n_active,
                                                          const int32_t *__restrict__ active,
                                                          const int32_t *__restrict__ offsets) {
  using S = Shape<2, MTX>;
  constexpr int kS = S::kStages;
  constexpr int kD = kS - 1;  // stages in flight ahead of the one in use
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kS * S::kSlot + kMetaBytes];
  unsigned char *stages = lds;
  unsigned char *meta = lds + kS * S::kSlot;

  // Routing lists into LDS and the barrier release base. Every load is issued
  // before the first value is used, so that the lists cost one round trip to
  // memory, not one per list, and no load or store sits behind a branch (the
  // compiler would sink the load into it): buffer loads past a list's end
  // return zero, every LDS entry of the lists is written (entries past the
  // active ones are never read), and the offsets' last rounds clamp to entry
  // kMaxE, which all their lanes then write with the same value.
  constexpr int kOffRounds = (kMaxE + 1 + kThreads - 1) / kThreads;
  constexpr int kActRounds = kMaxE / kThreads;
  constexpr int kPairRounds = kMaxPairs / kThreads;
  static_assert(kMaxE % kThreads == 0 && kMaxPairs % kThreads == 0, "list rounds");
  const __amdgpu_buffer_rsrc_t r_off = make_rsrc(offsets, uint32_t(p.E + 1) * 4u);
  const __amdgpu_buffer_rsrc_t r_act = make_rsrc(active, uint32_t(p.E) * 4u);
  const __amdgpu_buffer_rsrc_t r_tok = make_rsrc(p.pair_token, uint32_t(p.P) * 4u);
  const __amdgpu_buffer_rsrc_t r_slot = make_rsrc(p.pair_slot, uint32_t(p.P) * 4u);
  const uint32_t rel_base = release_base(p.sync);
  const int nact = n_active[0];
  int32_t offv[kOffRounds], actv[kActRounds], tokv[kPairRounds], slotv[kPairRounds];
#pragma unroll
  for (int r = 0; r < kOffRounds; ++r)
    offv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_off, min(int(threadIdx.x) + r * kThreads, kMaxE) * 4, 0, 0);
#pragma unroll
  for (int r = 0; r < kActRounds; ++r)
    actv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_act, (int(threadIdx.x) + r * kThreads) * 4, 0, 0);
#pragma unroll
  for (int r = 0; r < kPairRounds; ++r) {
    const int o = (int(threadIdx.x) + r * kThreads) * 4;
    tokv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_tok, o, 0, 0);
    slotv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_slot, o, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < kOffRounds; ++r)
    reinterpret_cast<int16_t *>(meta + kMetaOff)[min(int(threadIdx.x) + r * kThreads, kMaxE)] = int16_t(offv[r]);
#pragma unroll
  for (int r = 0; r < kActRounds; ++r)
    reinterpret_cast<int16_t *>(meta + kMetaAct)[threadIdx.x + r * kThreads] = int16_t(actv[r]);
#pragma unroll
  for (int r = 0; r < kPairRounds; ++r) {
    const int i = int(threadIdx.x) + r * kThreads;
    meta[kMetaTok + i] = uint8_t(tokv[r]);
    reinterpret_cast<int16_t *>(meta + kMetaRow)[i] = int16_t(tokv[r] * p.k + slotv[r]);
  }
  uint32_t *fill = reinterpret_cast<uint32_t *>(meta + kMetaFill);
  for (int t = threadIdx.x; t < p.B; t += kThreads) fill[t] = 0;
  __syncthreads();
  const int total = reinterpret_cast<const int16_t *>(meta + kMetaOff)[nact];
  // Filled slots of each token = its pairs in the list.
  for (int i = threadIdx.x; i < total; i += kThreads) atomicAdd(fill + meta[kMetaTok + i], 1u);
  __syncthreads();
  // Filled slots of each 16-token group: the count that completes it.
  if (threadIdx.x < kTokGroups) {
    uint32_t gs = 0;
    for (int t = threadIdx.x * kTokGroup; t < min(p.B, (threadIdx.x + 1) * kTokGroup); ++t) gs += fill[t];
    reinterpret_cast<uint32_t *>(meta + kMetaGFill)[threadIdx.x] = gs;
  }
  __syncthreads();
  zero_empty_groups(p, meta);

  // The gate/up split for this many active experts, chosen on the host
  // (plan_gate_up): stages of kBK rows per d slice, all of d for whole tiles.
  if constexpr (MTX < 4) {
    const uint32_t e = (up.e2[nact >> 1] >> (16 * (nact & 1))) & 0xFFFFu;
    p.slices = int(e >> 8);
    p.slice_rows = p.slices == 1 ? p.d : int(e & 0xFFu) * kBK;
  } else {
    // 64-token passes: the same rule with the planned slices, decided here
    // (reading the table slowed this instantiation's stage loop by 4-6%).
    const int G = int(gridDim.x);
    const int up_tiles = nact * ((p.I + kStripCols - 1) / kStripCols);
    bool whole;
    if (up_tiles <= G) {
      whole = 5 * up_tiles >= 3 * G;
    } else {
      const int whole_span = ((up_tiles + G - 1) / G) * ((p.d + kBK - 1) / kBK);
      const int sliced_span = ((up_tiles * p.slices + G - 1) / G) * (p.slice_rows / kBK) + kSliceCost;
      whole = p.slices == 1 || whole_span <= sliced_span;
    }
    if (whole) {
      p.slices = 1;
      p.slice_rows = p.d;
    }
  }

  const Stream<MTX> st(p, lds_addr(meta));
  Cursor cons;
  cons.per_up = ((p.I + kStripCols - 1) / kStripCols) * p.slices;
  cons.per_dn = (p.d + 2 * kStripCols - 1) / (2 * kStripCols);
  cons.n_up = nact * cons.per_up;
  cons.n_items = cons.n_up + nact * cons.per_dn;
  cons.item = blockIdx.x;
  st.decode(cons);
  Cursor prod = cons;

  // Prologue: kD stages in flight (gate/up only: down stages wait for h).
  // `issued` counts the stages issued so far.
  int issued = 0;
  for (int s = 0; s < kD; ++s) {
    if (!prod.valid || !prod.up) break;
    st.issue(prod, stages + s * S::kSlot);
    ++issued;
    st.advance(prod);
  }

  Acc acc;
  clear(acc);
  const uint32_t base = lds_addr(stages);
  bool h_ready = false;
  for (int s = 0; cons.valid; ++s) {
    if (!cons.up && !h_ready) {
      change_to_down<MTX>(p, st, prod, issued, s, stages, total, rel_base);
      h_ready = true;
    }
    // Stage s must have landed; the stages issued after it may stay in flight
    // (S::kCopies copies per wave each).
    const int newer = issued - s - 1;
    switch (newer < kD - 1 ? newer : kD - 1) {
      case 0: wait_barrier<0>(); break;
      case 1: wait_barrier<1 * S::kCopies>(); break;
      case 2: wait_barrier<(kD - 1 >= 2 ? 2 : 0) * S::kCopies>(); break;
      default: wait_barrier<(kD - 1 >= 3 ? 3 : 0) * S::kCopies>(); break;
    }
    // Every wave is past stage s-1, so its slot takes stage s+kD, whose
    // copies are issued in two halves during the compute of stage s.
    const bool fill = prod.valid && (prod.up || h_ready);
    unsigned char *fslot = stages + ((s + kD) % kS) * S::kSlot;
    compute_stage<MTX>(base + uint32_t((s % kS) * S::kSlot), st.trc, st.xrd, st.tp(cons), acc,
                       [&](int half) {
                         if (fill) st.issue_half(prod, fslot, half);
                       });
    if (fill) {
      ++issued;
      st.advance(prod);
    }
    if (cons.kst == cons.nst - 1) {
      epilogue<MTX>(cons, p, st.meta, st.wave, st.lane, acc);
      clear(acc);
      if (!cons.up) finish_down(cons, p, meta, st.wave, st.lane);
    }
    st.advance(cons);
  }
  if (!h_ready) change_to_down<MTX>(p, st, prod, issued, 0, stages, total, rel_base);  // no down items here
}

// ------------------------------------------------------------- combine (f32)
// y[t] = sum over slots j in order of w[t,j] * part[pair of (t,j)] (empty
// slots skipped).
__global__ __launch_bounds__(kThreads) void combine_f32_kernel(const float *__restrict__ part,
                                                               const int32_t *__restrict__ pair_of_slot,
                                                               const int32_t *__restrict__ topk_ids,
                                                               const float *__restrict__ topk_w,
                                                               int B, int d, int k, float *__restrict__ y) {
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
  *reinterpret_cast<float4 *>(y + size_t(t) * d + c) = acc;
}

// ----------------------------------------------------------- float32 path
// Small layers. A 1024-thread workgroup owns one (pair, 64-column block):
// row group r (16 of them) adds rows r, r+16, ... of each column with
// coalesced row loads; the 16 partial sums are then added in order.
constexpr int kF32Threads = 1024;
constexpr int kF32Cols = 64;
constexpr int kF32Groups = kF32Threads / kF32Cols;

// grid = (ceil(I/64), B*k): h[pair] = SiLU(x G) * (x U).
__global__ __launch_bounds__(kF32Threads) void up_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wg, const float *__restrict__ wu, int d,
    int I, int k, const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_token, const int32_t *__restrict__ pair_slot,
    const int32_t *__restrict__ topk_ids, float *__restrict__ h, int32_t *__restrict__ pair_of_slot) {
  __shared__ float red[2][kF32Groups][kF32Cols];
  const int pr = blockIdx.y;
  if (pr >= offsets[n_active[0]]) return;  // whole workgroup
  const int tx = threadIdx.x % kF32Cols, ty = threadIdx.x / kF32Cols;
  const int c = blockIdx.x * kF32Cols + tx;
  const int t = pair_token[pr];
  const int slot = t * k + pair_slot[pr];
  const int e = topk_ids[slot];
  if (blockIdx.x == 0 && threadIdx.x == 0) pair_of_slot[slot] = pr;
  float g = 0.f, u = 0.f;
  if (c < I) {
    const float *xr = x + size_t(t) * d;
    const float *G = wg + size_t(e) * d * I + c;
    const float *U = wu + size_t(e) * d * I + c;
#pragma unroll 4
    for (int i = ty; i < d; i += kF32Groups) {
      g = fmaf(xr[i], G[size_t(i) * I], g);
      u = fmaf(xr[i], U[size_t(i) * I], u);
    }
  }
  red[0][ty][tx] = g;
  red[1][ty][tx] = u;
  __syncthreads();
  if (ty == 0 && c < I) {
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int r = 0; r < kF32Groups; ++r) {
      gs += red[0][r][tx];
      us += red[1][r][tx];
    }
    h[size_t(pr) * I + c] = silu(gs) * us;
  }
}

// grid = (ceil(d/64), B*k): part[pair] = h D.
__global__ __launch_bounds__(kF32Threads) void down_f32_kernel(
    const float *__restrict__ h, const float *__restrict__ wd, int d, int I, int k,
    const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_token, const int32_t *__restrict__ pair_slot,
    const int32_t *__restrict__ topk_ids, float *__restrict__ part) {
  __shared__ float red[kF32Groups][kF32Cols];
  const int pr = blockIdx.y;
  if (pr >= offsets[n_active[0]]) return;  // whole workgroup
  const int tx = threadIdx.x % kF32Cols, ty = threadIdx.x / kF32Cols;
  const int c = blockIdx.x * kF32Cols + tx;
  const int e = topk_ids[pair_token[pr] * k + pair_slot[pr]];
  float acc = 0.f;
  if (c < d) {
    const float *hr = h + size_t(pr) * I;
    const float *D = wd + size_t(e) * I * d + c;
#pragma unroll 4
    for (int i = ty; i < I; i += kF32Groups) acc = fmaf(hr[i], D[size_t(i) * d], acc);
  }
  red[ty][tx] = acc;
  __syncthreads();
  if (ty == 0 && c < d) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kF32Groups; ++r) s += red[r][tx];
    part[size_t(pr) * d + c] = s;
  }
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

// Gate/up split for every possible active-expert count n (the count is only
// known on the device). A gate/up tile is (active expert, 64-column strip of
// I). Whole-d tiles when the tiles fill enough of the grid to keep HBM busy:
// each tile then forms its h columns itself and the grid meets once.
// Otherwise slices of d spread the gate/up work over the grid and h is
// formed from their partial sums between two grid barriers. With more tiles
// than workgroups, the path whose busiest workgroup streams fewer stages
// wins, the sliced one paying kSliceCost stages for its h phase and second
// barrier (a few tiles past the grid would otherwise double the phase). A
// sliced split takes the slice count, 2 up to the planned one (whose partial
// sums the workspace holds), whose busiest workgroup streams the fewest
// stages, ties to fewer slices (fewer, longer items and fewer partial sums
// to add: measured faster at 8-9 active experts). 72 tiles: 3 slices of 6
// stages make 216 items, where 4 slices of 4 make 288, two rounds of 4 for
// some workgroups.
static_assert(kMaxDim / kBK <= 255, "stages per slice fit a byte");
void plan_gate_up(const Params &p, int G, UpPlan &up) {
  for (uint32_t &w : up.e2) w = 0;
  const int nblk = ceil_div(p.d, kBK);
  const int strips = ceil_div(p.I, kStripCols);
  const int planned = p.slices;
  for (int n = 0; n <= p.E; ++n) {
    const int tiles = n * strips;
    int best_blk = nblk, best_span = 0x7fffffff;
    for (int sl = 2; sl <= planned; ++sl) {
      const int b = ceil_div(nblk, sl);
      const int span = ceil_div(tiles * ceil_div(nblk, b), G) * b;
      if (span < best_span) {
        best_span = span;
        best_blk = b;
      }
    }
    bool whole;
    if (planned == 1)
      whole = true;
    else if (tiles <= G)
      whole = 5 * tiles >= 3 * G;
    else
      whole = ceil_div(tiles, G) * nblk <= best_span + kSliceCost;
    const int blk = whole ? nblk : best_blk;
    const int slices = ceil_div(nblk, blk);
    up.e2[n >> 1] |= (uint32_t(blk) | uint32_t(slices) << 8) << (16 * (n & 1));
  }
}

template <int MTX>
void launch_ffn(int grid, const Params &p, const UpPlan &up, const moe_routing_t &r, hipStream_t s) {
  ffn_kernel<MTX><<<grid, kThreads, 0, s>>>(p, up, r.n_active, r.active_experts, r.expert_offsets);
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
    Params p{};
    p.x = static_cast<const uint16_t *>(x);
    p.W[0] = static_cast<const uint16_t *>(w_gate);
    p.W[1] = static_cast<const uint16_t *>(w_up);
    p.W[2] = static_cast<const uint16_t *>(w_down);
    p.B = B;
    p.d = d;
    p.E = E;
    p.I = I;
    p.k = k;
    p.slices = plan.up_slices;
    p.slice_rows = plan.up_slice_rows;
    p.P = P;
    p.gpart = reinterpret_cast<float *>(ws + plan.up_part);
    p.h = reinterpret_cast<uint16_t *>(ws + plan.h);
    p.part = part;
    p.y = static_cast<uint16_t *>(y);
    p.ids = r.topk_ids;
    p.w = r.topk_w;
    p.pair_token = r.pair_token;
    p.pair_slot = r.pair_slot;
    p.sync = reinterpret_cast<uint32_t *>(ws);
    p.grp_cnt = reinterpret_cast<uint32_t *>(ws + kGrpCntOffset);
    p.n_dstrips = ceil_div(d, 2 * kStripCols);
    // One workgroup per CU at most, so that the whole grid is resident and
    // the grid barriers cannot wait on a workgroup that has not started.
    const int items = max_active * (ceil_div(I, kStripCols) * plan.up_slices + ceil_div(d, 2 * kStripCols));
    const int cus = device_cus();
    const int grid = items < cus ? items : cus;
    UpPlan up;
    plan_gate_up(p, grid, up);
    // An expert has at most B tokens: A tiles of 16 * MTX rows cover them
    // (experts with more than 64 tokens take several passes).
    if (B <= 16)
      launch_ffn<1>(grid, p, up, r, s);
    else if (B <= 32)
      launch_ffn<2>(grid, p, up, r, s);
    else
      launch_ffn<4>(grid, p, up, r, s);
  } else {
    float *h = reinterpret_cast<float *>(ws + plan.h);
    up_f32_kernel<<<dim3(ceil_div(I, kF32Cols), P), kF32Threads, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(w_gate),
        static_cast<const float *>(w_up), d, I, k, r.n_active, r.expert_offsets, r.pair_token,
        r.pair_slot, r.topk_ids, h, pos);
    down_f32_kernel<<<dim3(ceil_div(d, kF32Cols), P), kF32Threads, 0, s>>>(
        h, static_cast<const float *>(w_down), d, I, k, r.n_active, r.expert_offsets,
        r.pair_token, r.pair_slot, r.topk_ids, part);
    combine_f32_kernel<<<ceil_div(B * (d / 4), kThreads), kThreads, 0, s>>>(
        part, pos, r.topk_ids, r.topk_w, B, d, k, static_cast<float *>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
