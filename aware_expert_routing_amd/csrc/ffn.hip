// Grouped SwiGLU expert FFN over the batch's active experts:
//   y[t] = sum_j w[t,j] * (SiLU(x_t G_e) * (x_t U_e)) D_e,  e = slot j's expert,
// reading only the weights of experts in the active list ("Lynx", Technical
// Summary 1: decode latency follows the number of distinct experts loaded;
// "Opportunistic Expert Activation", abstract: a decode step costs in
// proportion to how many different experts the batch switches on).
//
// bf16 path: one persistent kernel, one workgroup per CU.
//   * Work items: gate/up items (active expert x 64-column strip of I x slice
//     of d) come first, then down items (active expert x 128-column strip of
//     d x slice of I); workgroup b takes items b, b+G, b+2G, ... The gate/up
//     tiles are taken whole, split over d, or whole for the grid's full
//     rounds and split for the rest (a plan costed per active-expert count on
//     the host); when whole tiles fit one round with workgroups to spare, the
//     tiles of the slow strips (byte offset 384 mod 512 of a weight row) are
//     split in two over d, and in mixed plans they come last; down items are
//     split over I when few experts are active.
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
//   * A whole gate/up tile writes h = SiLU(g) * u from its accumulators; the
//     slices of a split tile store partial sums and the workgroup that counts
//     a tile's last slice forms its h. One grid barrier then separates
//     gate/up from down.
//   * A down pass adds its tokens to per-(16-token group, strip) counters;
//     the workgroup that completes a group's count forms y over that strip
//     for the group's tokens, adding the slots (and a slot's I slices) in
//     order (no float atomics: results are reproducible). Above 32 tokens it
//     queues the combine instead, and every workgroup drains the queue once
//     its down items are done.
// float32 path (small layers): plain dot products, 16 row groups per column.
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

// Measurement build only (compiled with -DMOE_PHASE_STAMPS into a separate
// library; the product build compiles all of this away): lane 0 of every
// workgroup records the 100 MHz s_memrealtime counter at the phase
// boundaries into stamps[workgroup][64]: 0 start, 1 routing lists in LDS,
// 2 first stage computed, 3 gate/up done, 4 past the first grid barrier,
// 5 first down stages landed, 6 a down item's last stage computed, 7 its
// rows stored, 8 counted, 9 a combine done, 10 end; 16 + s: stage s passed
// its wait (bit 63 set for a down stage), s < 48.
#ifdef MOE_PHASE_STAMPS
#define MOE_STAMP(i)                                                                    \
  do {                                                                                  \
    if (threadIdx.x == 0 && p.stamps) p.stamps[blockIdx.x * 64 + (i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define MOE_STAGE_STAMP(s, down)                                                          \
  do {                                                                                    \
    if (threadIdx.x == 0 && p.stamps && (s) < 48)                                         \
      p.stamps[blockIdx.x * 64 + 16 + (s)] =                                              \
          __builtin_amdgcn_s_memrealtime() | ((down) ? (1ull << 63) : 0ull);              \
  } while (0)
#else
#define MOE_STAMP(i) \
  do {           \
  } while (0)
#define MOE_STAGE_STAMP(s, down) \
  do {                       \
  } while (0)
#endif

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
// SC0 alone: the load skips the compute unit's L1 and reads the XCD's L2,
// which holds the latest data stored from this XCD.
constexpr int kPolicyL2 = 1;

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

// Reads v at this point (an empty asm with v as input), so that the compiler
// waits here for the load that wrote it. Cold code inside the stage loop
// loads values that it may then read only on some paths; a register whose
// load the compiler cannot see completed on every path stays pending around
// the loop, and the compiler then waits for it (and for every weight copy
// issued before it) wherever the stage loop reuses that register.
__device__ __forceinline__ void consume(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void consume(float4 v) { asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)); }

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
constexpr int kSyncErr = int(kSyncErrOffset / 4);
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

// Gate/up split for `tiles` gate/up tiles (active expert, 64-column strip of
// I) of nblk stages each on G workgroups, as an UpPlan entry: stages per
// slice | slices << 8 | kUpMixed. Three forms:
//   whole    every tile takes all of d (h formed in its epilogue);
//   sliced   every tile is split into 2 up to `planned` d slices (the
//            partial sums the workspace holds);
//   mixed    the tiles of whole rounds of the grid are taken whole and the
//            rest (fewer than G) are split so that every slice item gets a
//            workgroup of its own in the last round.
// The cost of a form is its busiest workgroup's stages, plus kFinishStages
// per sliced item: after a sliced item a workgroup waits for its partial sums
// to be stored and counted, and the workgroup completing a tile forms its h,
// a few round trips to memory under full load (about four stages' time,
// measured). The cheapest wins, ties to whole tiles and then to fewer slices
// (fewer partial sums to store and add). More split tiles than tile
// counters are not split.
constexpr int kFinishStages = 4;
constexpr uint32_t kUpMixed = 1u << 15;
inline uint32_t plan_split(int tiles, int nblk, int planned, int G) {
  uint32_t best = uint32_t(nblk) | (1u << 8);
  int best_cost = (tiles + G - 1) / G * nblk;
  for (int sl = 2; sl <= planned && tiles <= kMaxTileCounters; ++sl) {
    const int b = (nblk + sl - 1) / sl, ns = (nblk + b - 1) / b;
    const int cost = (tiles * ns + G - 1) / G * (b + kFinishStages);
    if (cost < best_cost) {
      best_cost = cost;
      best = uint32_t(b) | uint32_t(ns) << 8;
    }
  }
  const int whole = tiles / G * G, rest = tiles - whole;
  for (int sl = 2; sl <= planned && whole > 0 && rest > 0; ++sl) {
    const int b = (nblk + sl - 1) / sl, ns = (nblk + b - 1) / b;
    if (rest * ns > G) break;
    const int cost = whole / G * nblk + b + kFinishStages;
    if (cost < best_cost) {
      best_cost = cost;
      best = uint32_t(b) | uint32_t(ns) << 8 | kUpMixed;
    }
  }
  return best;
}

struct Params {
  const uint16_t *x;          // [B, d]
  const uint16_t *W[3];       // G, U: [E, d, I]; D: [E, I, d]
  int B, d, E, I, k;
  int slices;                 // most gate/up d slices (the partial sums the workspace holds)
  int n_ustrips;              // 64-column strips of I
  int P;                      // B * k
  float *gpart;               // [slices][2][P][I] gate/up partial sums by pair
  uint16_t *h;                // [P][I] SiLU(g) * u by pair
  float *part;                // [P][d] down-projection rows by token slot t*k+j
  uint16_t *y;                // [B][d]
  const float *w;             // [B][k]
  const int32_t *pair_token;  // [P]
  const int32_t *pair_slot;   // [P]
  uint32_t *sync;             // grid-barrier words
#ifdef MOE_PHASE_STAMPS
  uint64_t *stamps;           // measurement build: phase stamps
#endif
  uint32_t *grp_cnt;          // per (strip, token group): slots counted, one 128-byte line each
  uint32_t *tile_cnt;         // per gate/up tile (sliced path): d slices counted
  int n_dstrips;              // 128-column strips of d
  int dslices;                // most down I slices (the partial rows the workspace holds)
  uint32_t *queue;            // B > 32: combine queue (pop, push, done words; entries)
};

// The work split of one launch, chosen on the device from the active-expert
// count (Params stays as the launch passed it).
struct Split {
  int slices, slice_rows;    // gate/up: d slices of a split tile, rows per slice
  int up_whole;              // gate/up tiles taken whole (the first ones; h formed in the epilogue)
  int dslices, dslice_rows;  // down: I slices of an item (1: all of I), rows per slice
  int slow;                  // 1: the tiles of strips 4q+3 come after the others' (below)
  int nfast;                 // with slow: the tiles of the other strips, which come first
};

// By active-expert count: gate/up stages of kBK rows per d slice (all of d
// for whole tiles). A kernel argument of its own, never written, so that the
// kernel reads the entry it needs from the argument segment.
struct UpPlan {
  // Entry n in half n % 2 of word n / 2: stages per slice | slices << 8 |
  // kUpMixed (the tiles of whole rounds of the grid are taken whole).
  uint32_t e2[(kMaxE + 2) / 2];
};

// A position in a workgroup's stage sequence. The workgroup's items are
// b, b+G, b+2G, ... of one list: gate/up items first (expert, 64-column strip
// of I, slice of d), then down items (expert, 128-column strip of d, all of
// I). Every stage holds two weight tiles (G and U, or two adjacent 64-column
// tiles of D) and the A tile of the same reduction rows (x rows gathered by
// token, or h rows by pair). All fields are wave-uniform.
struct Cursor {
  int item, n_items, n_up, per_dn;
  int e, p0, T, strip, ks, row0, nrows, nst, npass, pass, kst;
  bool valid, up;
};

template <int MTX>
struct Stream {
  using S = Shape<2, MTX>;
  const Params &p;
  const Split sp;
  uint32_t meta;            // LDS address of the routing lists
  int wave, lane, g, j;
  uint32_t wv_up[4];        // weight copy offsets within a stage (row stride I)
  uint32_t wv_dn[4];        // the same for D (row stride d)
  uint32_t trc[2];          // transposing-read offsets within a weight tile
  uint32_t xrd;             // A-fragment read offset within a k-step sub-tile

  __device__ __forceinline__ Stream(const Params &pp, const Split &s, uint32_t meta_addr)
      : p(pp), sp(s), meta(meta_addr) {
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
    // The fields are computed in locals and stored once below (stores of
    // different fields in the two branches were merged through a pointer
    // phi, which kept the cursor in scratch memory).
    int a, strip, ks, row0, nrows;
    if (c.up) {
      // Whole tiles first (ks = -1), then the d slices of each split tile.
      int tile;
      if (c.item < sp.up_whole) {
        tile = c.item;
        ks = -1;
        row0 = 0;
        nrows = p.d;
      } else {
        const int j = c.item - sp.up_whole;
        const int ts = j / sp.slices;
        tile = sp.up_whole + ts;
        ks = j - ts * sp.slices;
        row0 = ks * sp.slice_rows;
        nrows = min(sp.slice_rows, p.d - row0);
      }
      // Tile -> (expert, strip). Normally tile = expert * strips + strip.
      // With sp.slow the first sp.nfast tiles take, expert by expert, the
      // strips other than 4q+3 (strip r + r/3 for the r-th of them) and the
      // rest the strips 4q+3. Selects rather than branches: this code is
      // inlined into the stage loop, whose scalar registers are scarce.
      const int f = sp.slow, ns = p.n_ustrips >> 2;
      const bool slow_group = tile >= sp.nfast;
      const int u = f && slow_group ? tile - sp.nfast : tile;
      const int dv = f ? (slow_group ? ns : p.n_ustrips - ns) : p.n_ustrips;
      a = u / dv;
      const int r = u - a * dv;
      strip = f ? (slow_group ? 4 * r + 3 : r + r / 3) : r;
    } else {
      const int jd = c.item - c.n_up;
      a = jd / c.per_dn;
      const int rem = jd - a * c.per_dn;
      strip = rem / sp.dslices;
      ks = rem - strip * sp.dslices;
      row0 = ks * sp.dslice_rows;
      nrows = min(sp.dslice_rows, p.I - row0);
    }
    c.strip = strip;
    c.ks = ks;
    c.row0 = row0;
    c.nrows = nrows;
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
  template <bool UP>
  __device__ __forceinline__ uint32_t xvoff(const Cursor &c, int h) const {
    const int m = 16 * h + (lane >> 2);
    const int T = tp(c);
    const int pr = c.p0 + c.pass * kMaxTok + (m < T ? m : T - 1);
    const int lc = (lane & 3) ^ swz_x(m);
    const uint32_t kofs = uint32_t(wave * 32 + lc * 8);
    if constexpr (UP) return (uint32_t(lds_u8(meta + kMetaTok + pr)) * uint32_t(p.d) + kofs) * 2u;
    return (uint32_t(pr) * uint32_t(p.I) + kofs) * 2u;
  }

  // The A-tile copies of stage c (MTX per wave): x rows by token for gate/up,
  // h rows by pair for down (device scope: other workgroups wrote h).
  template <bool UP>
  __device__ __forceinline__ void issue_a(const Cursor &c, unsigned char *slot) const {
    unsigned char *dst = slot + 2 * kWTile + wave * S::kXSub;
    const uint32_t xsoff = uint32_t(c.row0 + c.kst * kBK) * 2u;
    if constexpr (UP) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.x, uint32_t(p.B) * uint32_t(p.d) * 2u);
#pragma unroll
      for (int h = 0; h < MTX; ++h) dma16(ra, dst + h * 1024, xvoff<true>(c, h), xsoff);
    } else {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.h, uint32_t(p.P) * uint32_t(p.I) * 2u);
#pragma unroll
      for (int h = 0; h < MTX; ++h) dma16<kPolicyDevice>(ra, dst + h * 1024, xvoff<false>(c, h), xsoff);
    }
  }

  // The weight copies of down stage c that wave `vw` normally issues (4 per
  // tile), issued by this wave: used while wave 0 is busy at the grid barriers.
  __device__ __forceinline__ void issue_dn_weights_as(const Cursor &c, unsigned char *slot, int vw) const {
    const size_t base = size_t(c.e) * p.I * p.d;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p.W[2] + base, uint32_t(p.I) * uint32_t(p.d) * 2u);
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      const uint32_t soff = (uint32_t(c.row0 + c.kst * kBK) * uint32_t(p.d) +
                             uint32_t((2 * c.strip + mat) * kStripCols)) * 2u;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int rr = 8 * (vw + 4 * h) + (lane >> 3);
        const uint32_t voff = uint32_t(rr) * uint32_t(p.d) * 2u + uint32_t((lane & 7) ^ swz_w(rr)) * 16u;
        dma16<kPolicyStream>(r, slot + mat * kWTile + (vw + 4 * h) * 1024, voff, soff);
      }
    }
  }

  // Issues half of this wave's copies of stage c (a gate/up stage when UP,
  // else a down stage) into `slot`: half 0 the first weight tile and the A
  // tile, half 1 the second weight tile (S::kCopies per wave in all).
  template <bool UP>
  __device__ __forceinline__ void issue_half(const Cursor &c, unsigned char *slot, int half) const {
    if constexpr (UP) {
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
      const uint32_t soff = (uint32_t(c.row0 + c.kst * kBK) * uint32_t(p.d) +
                             uint32_t((2 * c.strip + half) * kStripCols)) * 2u;
#pragma unroll
      for (int h = 0; h < 4; ++h) dma16<kPolicyStream>(r, slot + half * kWTile + (wave + 4 * h) * 1024, wv_dn[h], soff);
    }
    if (half == 0) issue_a<UP>(c, slot);
  }
  // Issues every copy of gate/up stage c into `slot`.
  __device__ __forceinline__ void issue_up(const Cursor &c, unsigned char *slot) const {
    issue_half<true>(c, slot, 0);
    issue_half<true>(c, slot, 1);
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

// Operand fragments of the four k-steps of a stage (pairs K = 0, 1 of steps
// J = 0, 1; k-step ks = 2K + J), read from LDS by one inline-assembly block
// that waits once, so that all the reads of a stage overlap. Per k-step:
//   B fragments (column 16*wave + j, rows 32ks + 8g .. +7 of both weight
//   tiles): four transposing reads at the lane's offsets b0 and b1 (rows
//   8g + 4h + j/4 of the k-step), in tile 0 and in tile 1 (kWTile further),
//   into t[K][J][0..3]; the read gives lane j of a 16-lane group element j of
//   the four rows its group's lanes point at (lane 4r+q points at row r,
//   columns 4q..4q+3);
//   A fragments: NA reads of 16 bytes at xa[mt] + ks * XS (row tile mt),
//   into a[K][J][mt].
#define MOE_TR4(K, J)                                                          \
  "ds_read_b64_tr_b16 %[t" #K #J "0], %[B0] offset:%[ob" #K #J "]\n\t"         \
  "ds_read_b64_tr_b16 %[t" #K #J "1], %[B1] offset:%[ob" #K #J "]\n\t"         \
  "ds_read_b64_tr_b16 %[t" #K #J "2], %[B0] offset:%[ow" #K #J "]\n\t"         \
  "ds_read_b64_tr_b16 %[t" #K #J "3], %[B1] offset:%[ow" #K #J "]\n\t"
#define MOE_TR_READS MOE_TR4(0, 0) MOE_TR4(0, 1) MOE_TR4(1, 0) MOE_TR4(1, 1)
#define MOE_A(K, J, M) "ds_read_b128 %[a" #K #J #M "], %[X" #M "] offset:%[oa" #K #J "]\n\t"
#define MOE_A_READS(M) MOE_A(0, 0, M) MOE_A(0, 1, M) MOE_A(1, 0, M) MOE_A(1, 1, M)
#define MOE_T_OUT4(K, J)                                                                 \
  [t##K##J##0] "=&v"(t[K][J][0]), [t##K##J##1] "=&v"(t[K][J][1]), [t##K##J##2] "=&v"(t[K][J][2]), \
  [t##K##J##3] "=&v"(t[K][J][3])
#define MOE_T_OUTS MOE_T_OUT4(0, 0), MOE_T_OUT4(0, 1), MOE_T_OUT4(1, 0), MOE_T_OUT4(1, 1)
#define MOE_A_OUTS(M)                                                                    \
  [a00##M] "=&v"(a[0][0][M]), [a01##M] "=&v"(a[0][1][M]), [a10##M] "=&v"(a[1][0][M]),   \
  [a11##M] "=&v"(a[1][1][M])
#define MOE_OFF(K, J)                                                                    \
  [ob##K##J] "i"((2 * K + J) * 32 * kRowBytes), [ow##K##J] "i"((2 * K + J) * 32 * kRowBytes + kWTile), \
  [oa##K##J] "i"((2 * K + J) * XS)
#define MOE_INS [B0] "v"(b0), [B1] "v"(b1), MOE_OFF(0, 0), MOE_OFF(0, 1), MOE_OFF(1, 0), MOE_OFF(1, 1)

template <int NA, int XS>
struct StageFrags;

template <int XS>
struct StageFrags<1, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][2][4], bf16x8_t (&a)[2][2][4]) {
    asm volatile(MOE_TR_READS MOE_A_READS(0) "s_waitcnt lgkmcnt(0)"
                 : MOE_T_OUTS, MOE_A_OUTS(0)
                 : MOE_INS, [X0] "v"(xa[0]));
  }
};
template <int XS>
struct StageFrags<2, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][2][4], bf16x8_t (&a)[2][2][4]) {
    asm volatile(MOE_TR_READS MOE_A_READS(0) MOE_A_READS(1) "s_waitcnt lgkmcnt(0)"
                 : MOE_T_OUTS, MOE_A_OUTS(0), MOE_A_OUTS(1)
                 : MOE_INS, [X0] "v"(xa[0]), [X1] "v"(xa[1]));
  }
};
template <int XS>
struct StageFrags<3, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][2][4], bf16x8_t (&a)[2][2][4]) {
    asm volatile(MOE_TR_READS MOE_A_READS(0) MOE_A_READS(1) MOE_A_READS(2) "s_waitcnt lgkmcnt(0)"
                 : MOE_T_OUTS, MOE_A_OUTS(0), MOE_A_OUTS(1), MOE_A_OUTS(2)
                 : MOE_INS, [X0] "v"(xa[0]), [X1] "v"(xa[1]), [X2] "v"(xa[2]));
  }
};
template <int XS>
struct StageFrags<4, XS> {
  __device__ __forceinline__ static void read(uint32_t b0, uint32_t b1, const uint32_t (&xa)[4],
                                              long (&t)[2][2][4], bf16x8_t (&a)[2][2][4]) {
    asm volatile(MOE_TR_READS MOE_A_READS(0) MOE_A_READS(1) MOE_A_READS(2) MOE_A_READS(3)
                 "s_waitcnt lgkmcnt(0)"
                 : MOE_T_OUTS, MOE_A_OUTS(0), MOE_A_OUTS(1), MOE_A_OUTS(2), MOE_A_OUTS(3)
                 : MOE_INS, [X0] "v"(xa[0]), [X1] "v"(xa[1]), [X2] "v"(xa[2]), [X3] "v"(xa[3]));
  }
};
#undef MOE_TR4
#undef MOE_TR_READS
#undef MOE_A
#undef MOE_A_READS
#undef MOE_T_OUT4
#undef MOE_T_OUTS
#undef MOE_A_OUTS
#undef MOE_OFF
#undef MOE_INS

// MFMA work of one stage: every fragment read at once, then the two pairs
// of k-steps; hook(kp) runs before pair kp (the loop issues half of a later
// stage's copies there, so that the copies enter the memory pipeline while
// this stage computes). One LDS wait per stage instead of one per pair:
// bit-identical outputs, FFN spec-decode B=64 topk 88.6 -> 87.7 us,
// Qwen3-235B-shaped B=64 oea(4) 228.9 -> 227.7, the 16-token shapes within
// 0.2 us either way.
template <int MTX, int NA, class Hook>
__device__ __forceinline__ void mfma_stage(uint32_t slot, uint32_t xslot, const uint32_t (&trc)[2],
                                           uint32_t xrd, Acc &acc, const Hook &hook) {
  constexpr int XS = Shape<2, MTX>::kXSub;
  static_assert(kKSteps == 4, "two pairs of k-steps per stage");
  const uint32_t b0 = slot + trc[0], b1 = slot + trc[1];
  uint32_t xa[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) xa[mt] = xslot + uint32_t(mt * 1024) + xrd;
  hook(0);
  long t[2][2][4];
  bf16x8_t a[2][2][4];
  StageFrags<NA, XS>::read(b0, b1, xa, t, a);
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    if (kp == 1) hook(1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bf16x8_t b[2];
      __builtin_memcpy(&b[0], &t[kp][q][0], 8);
      __builtin_memcpy(reinterpret_cast<char *>(&b[0]) + 8, &t[kp][q][1], 8);
      __builtin_memcpy(&b[1], &t[kp][q][2], 8);
      __builtin_memcpy(reinterpret_cast<char *>(&b[1]) + 8, &t[kp][q][3], 8);
#pragma unroll
      for (int mt = 0; mt < NA; ++mt)
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
          acc.mf[mat][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kp][q][mt], b[mat], acc.mf[mat][mt], 0, 0, 0);
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
// A pass has at most 16 * MTX tokens. UP: c is a gate/up item.
template <int MTX, bool UP>
__device__ __forceinline__ void epilogue(const Cursor &c, const Params &p, uint32_t meta, int wave,
                                         int lane, Acc &acc) {
  const int g = lane >> 4, j = lane & 15;
  const int T = min(kMaxTok, c.T - c.pass * kMaxTok);
  const int pbase = c.p0 + c.pass * kMaxTok;
  if (UP && c.ks < 0) {
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
  if constexpr (UP) {
    ld = p.I;
    col0 = col1 = c.strip * kStripCols + 16 * wave + j;
    dst0 = p.gpart + size_t(c.ks * 2) * p.P * p.I;
    dst1 = dst0 + size_t(p.P) * p.I;
  } else {
    ld = p.d;
    col0 = 2 * c.strip * kStripCols + 16 * wave + j;
    col1 = col0 + kStripCols;
    dst0 = dst1 = p.part + size_t(c.ks) * p.P * p.d;
  }
  const bool ok0 = col0 < ld, ok1 = col1 < ld;
#pragma unroll
  for (int t4 = 0; t4 < MTX; ++t4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * t4 + 4 * g + i;
      if (m < T) {
        const size_t row = size_t(UP ? pbase + m : lds_i16(meta + kMetaRow + 2 * (pbase + m))) * ld;
        if (ok0) st_dev(dst0 + row + col0, acc.mf[0][t4][i]);
        if (ok1) st_dev(dst1 + row + col1, acc.mf[1][t4][i]);
      }
    }
}

// End of a gate/up item of the sliced path (every pass of it has stored its
// partial sums of g and u, device scope). The item counts itself on its
// tile's counter; the workgroup that brings the count to the number of d
// slices forms h = SiLU(g) * u for the tile's 64 columns and every token of
// the expert from the slices' partial sums, added in slice order, and puts
// the counter back to zero. So h is complete once every workgroup has
// finished its gate/up items, and one grid barrier separates gate/up from
// down. `flag` is an int in LDS.
__device__ __forceinline__ void finish_up(const Cursor &c, const Params &p, const Split &sp, int *flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    // Split tiles are counted in order: counter (item - up_whole) / slices.
    uint32_t *cnt = p.tile_cnt + size_t((c.item - sp.up_whole) / sp.slices) * kTileCntStride;
    const uint32_t before = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before + 1 == uint32_t(sp.slices);
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  const uint32_t blk = uint32_t(p.P) * uint32_t(p.I) * 4u;  // bytes of one [P][I] block
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p.gpart, uint32_t(sp.slices) * 2u * blk);
  const int col0 = c.strip * kStripCols;
  for (int u = threadIdx.x; u < c.T * (kStripCols / 4); u += kThreads) {
    const int m = u / (kStripCols / 4);
    const int col = col0 + (u - m * (kStripCols / 4)) * 4;  // I % 8 == 0: col < I means col + 3 < I
    if (col >= p.I) continue;
    const uint32_t off = (uint32_t(c.p0 + m) * uint32_t(p.I) + uint32_t(col)) * 4u;
    // Slices past sp.slices load slice 0 again and are masked out: every
    // load is unconditional and read at once (consume).
    float4 gv[kUpMaxSlices], uv[kUpMaxSlices];
#pragma unroll
    for (int sl = 0; sl < kUpMaxSlices; ++sl) {
      const uint32_t so = uint32_t(sl < sp.slices ? sl : 0) * 2u * blk;
      gv[sl] = ld_dev4(r, off + so);
      uv[sl] = ld_dev4(r, off + so + blk);
    }
#pragma unroll
    for (int sl = 0; sl < kUpMaxSlices; ++sl) {
      consume(gv[sl]);
      consume(uv[sl]);
    }
    float4 g = make_float4(0, 0, 0, 0), v = make_float4(0, 0, 0, 0);
#pragma unroll
    for (int sl = 0; sl < kUpMaxSlices; ++sl) {
      const bool in = sl < sp.slices;
      const float4 a = in ? gv[sl] : make_float4(0, 0, 0, 0);
      const float4 b = in ? uv[sl] : make_float4(0, 0, 0, 0);
      g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
      v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
    }
    const uint64_t o = uint64_t(f32_to_bf16(silu(g.x) * v.x)) |
                       (uint64_t(f32_to_bf16(silu(g.y) * v.y)) << 16) |
                       (uint64_t(f32_to_bf16(silu(g.z) * v.z)) << 32) |
                       (uint64_t(f32_to_bf16(silu(g.w) * v.w)) << 48);
    st_dev(reinterpret_cast<uint64_t *>(p.h + size_t(c.p0 + m) * p.I + col), o);
  }
}

// s_barrier without the wait for outstanding memory operations that
// __syncthreads adds: copies in flight stay in flight.
__device__ __forceinline__ void barrier_no_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Counter of (token group grp, down strip) on a 128-byte line of its own: a
// 64-bit word holding, over the passes counted so far, S0 = sum of run
// (bits 0-15: filled slots counted), S1 = sum of run * x (bits 16-31) and
// S2 = sum of run * x^2 (bits 32-63), x being the XCD each pass ran on. By
// Cauchy-Schwarz, S1^2 == S0 * S2 exactly when every pass ran on one XCD,
// which is then x = S1 / S0.
__device__ __forceinline__ uint64_t *group_counter(const Params &p, int grp, int strip) {
  return reinterpret_cast<uint64_t *>(p.grp_cnt + (size_t(strip) * kTokGroups + grp) * kCntStride);
}

// The XCD (accelerator complex die) this wave runs on: bits 3:0 of the
// XCC_ID hardware register.
__device__ __forceinline__ uint32_t xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u; }

// y over 128-column strip `strip` for the tokens of group grp: thread i takes
// token 16*grp + i/16 and columns 8*(i%16) .. +7 of the strip, adding
// w[t,j] * (part[0][t*k+j] + part[1][t*k+j] + ...) (the I slices' rows, in
// slice order) in slot order over the token's filled slots (fill[t] of
// them; a routing's empty slots trail its filled ones). Up to eight rows are
// loaded per round, every load of a round issued before the first use. The
// rows were stored with device-scope stores, which also update the L2 of the
// storing XCD; when every row of the group's strip came from this
// workgroup's XCD (`local`), they are read through that L2, else from the
// device-coherent level.
static_assert(kThreads == kTokGroup * (2 * kStripCols / 8), "one thread per token and 8 columns");
__device__ __forceinline__ float4 ld_part4(__amdgpu_buffer_rsrc_t r, uint32_t off, bool local) {
  const f32x4_t v = local ? __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kPolicyL2))
                          : __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kPolicyDevice));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void combine_group(const Params &p, int ds, const uint32_t *fill, int grp,
                                              int strip, bool local) {
  const int t = grp * kTokGroup + (threadIdx.x >> 4);
  const int col = strip * 2 * kStripCols + (threadIdx.x & 15) * 8;
  if (t >= p.B || col >= p.d) return;
  const int nf = int(fill[t]);
  const int per_round = max(1, 8 / ds);  // slots per round
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part, uint32_t(ds) * uint32_t(p.P) * uint32_t(p.d) * 4u);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nf; j0 += per_round) {
    const int nq = min(per_round, nf - j0) * ds;  // rows this round
    // Row q of the round: slot j0 + q / ds, I slice q % ds. Rows past nq
    // load row q = 0 again and are masked out: every load is unconditional
    // and read at once (consume).
    float w[8];
    float4 v[8][2];
    int jj = 0, ks = 0;  // q / ds and q % ds
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = q < nq;
      const int slot = t * p.k + j0 + (in ? jj : 0);
      w[q] = p.w[slot];
      const uint32_t off = ((uint32_t(in ? ks : 0) * uint32_t(p.P) + uint32_t(slot)) * uint32_t(p.d) + uint32_t(col)) * 4u;
      v[q][0] = ld_part4(rp, off, local);
      v[q][1] = ld_part4(rp, off + 16u, local);
      if (++ks == ds) {
        ks = 0;
        ++jj;
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      consume(w[q]);
      consume(v[q][0]);
      consume(v[q][1]);
    }
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = make_float4(0.f, 0.f, 0.f, 0.f);
    ks = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = q < nq;
      const bool last = ++ks == ds;  // the slot's last I slice
      if (last) ks = 0;
      const float4 a = in ? v[q][0] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 b = in ? v[q][1] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float wj = in ? w[q] : 0.f;
      s0.x += a.x; s0.y += a.y; s0.z += a.z; s0.w += a.w;
      s1.x += b.x; s1.y += b.y; s1.z += b.z; s1.w += b.w;
      if (in && last) {
        acc[0] = fmaf(wj, s0.x, acc[0]);
        acc[1] = fmaf(wj, s0.y, acc[1]);
        acc[2] = fmaf(wj, s0.z, acc[2]);
        acc[3] = fmaf(wj, s0.w, acc[3]);
        acc[4] = fmaf(wj, s1.x, acc[4]);
        acc[5] = fmaf(wj, s1.y, acc[5]);
        acc[6] = fmaf(wj, s1.z, acc[6]);
        acc[7] = fmaf(wj, s1.w, acc[7]);
      }
      if (last) {
        s0 = make_float4(0.f, 0.f, 0.f, 0.f);
        s1 = make_float4(0.f, 0.f, 0.f, 0.f);
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

// Combine queue words (Params::queue): pop index, push index, workgroups
// done, each on a 128-byte line, then the entries (strip << 8 | group) + 1.
constexpr int kQueuePop = 0;
constexpr int kQueuePush = 32;
constexpr int kQueueDone = 64;
constexpr int kQueueEnt = 96;

// End of a down pass (its rows stored by every wave). The pass adds, for
// each 16-token group it has tokens of, their number to the group's counter
// for the strip (one atomic per group, not per token: the atomics of one
// counter are served in turn). The workgroup that brings a counter to the
// group's number of filled slots resets it and forms y over the strip for
// the group (combine_group), or, with more than 32 tokens (QUEUED: up to 16
// groups per strip, which one workgroup would combine one round trip after
// another), pushes the (strip, group) combine onto the queue that every
// workgroup drains once its down items are done (drain_combines), so that a
// strip's groups are combined by different workgroups at once (each then
// waits one poll more; with two groups per strip that costs more than it
// saves). A count is taken only after this workgroup's stores have
// completed, so the last one finds every row of the group in place.
template <bool QUEUED>
__device__ __forceinline__ void finish_down(const Cursor &c, const Params &p, const Split &sp,
                                            unsigned char *meta, int wave, int lane) {
  const int T = min(kMaxTok, c.T - c.pass * kMaxTok);
  const int pbase = c.p0 + c.pass * kMaxTok;
  int32_t *last = reinterpret_cast<int32_t *>(meta + kMetaLast);
  int32_t *n_last = reinterpret_cast<int32_t *>(meta + kMetaNLast);
  const uint32_t *gfill = reinterpret_cast<const uint32_t *>(meta + kMetaGFill);
  MOE_STAMP(6);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  MOE_STAMP(7);
  if (wave == 0) {
    // The first lane of each run of lanes in one group adds the run's
    // length (an expert's tokens ascend, so a group is one run).
    const int grp = lane < T ? int(meta[kMetaTok + pbase + lane]) / kTokGroup : -1;
    const int prev = __shfl_up(grp, 1);
    const bool first = lane < T && (lane == 0 || prev != grp);
    const unsigned long long fb = __ballot(first);
    bool mine = false;
    int local = 0;
    if (first) {
      const unsigned long long above = lane == 63 ? 0ull : (fb >> (lane + 1));
      const uint64_t run = above ? __builtin_ctzll(above) + 1 : T - lane;
      const uint64_t x = xcd_id();
      const uint64_t add = run | ((run * x) << 16) | ((run * x * x) << 32);
      const uint64_t now = __hip_atomic_fetch_add(group_counter(p, grp, c.strip), add,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
      const uint64_t s0 = now & 0xFFFFu, s1 = (now >> 16) & 0xFFFFu, s2 = now >> 32;
      mine = s0 == gfill[grp] * uint32_t(sp.dslices);
      local = mine && s1 * s1 == s0 * s2 && s1 == s0 * x;
    }
    const unsigned long long b = __ballot(mine);
    if constexpr (QUEUED) {
      if (mine) {
        __hip_atomic_store(group_counter(p, grp, c.strip), uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t i = __hip_atomic_fetch_add(p.queue + kQueuePush, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.queue + kQueueEnt + i, uint32_t((c.strip << 8 | grp) + 1), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0) *n_last = 0;
    } else {
      if (mine) last[__builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(b), 0))] = grp | (local << 16);
      if (lane == 0) *n_last = __popcll(b);
    }
  }
  __syncthreads();
  MOE_STAMP(8);
  const int n = *n_last;
  for (int q = 0; q < n; ++q) {
    const int grp = last[q] & 0xFFFF;
    combine_group(p, sp.dslices, reinterpret_cast<const uint32_t *>(meta + kMetaFill), grp, c.strip,
                  (last[q] >> 16) != 0);
    if (threadIdx.x == 0)
      __hip_atomic_store(group_counter(p, grp, c.strip), uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (n) MOE_STAMP(9);
}

// The combine queue's consumer, run by every workgroup after its down items:
// it takes entries in order (one atomic on the pop index each) until every
// combine of the launch (128-column strips x token groups with a filled
// slot) has been taken, waits for each taken entry to be pushed (bounded
// polls; a wait that gives up sets the error word) and forms y for it. The
// last workgroup done puts the queue's indices back to zero; each entry is
// cleared by the workgroup that takes it.
__device__ __forceinline__ void drain_combines(const Params &p, int ds, unsigned char *meta) {
  const uint32_t *gfill = reinterpret_cast<const uint32_t *>(meta + kMetaGFill);
  int32_t *code_lds = reinterpret_cast<int32_t *>(meta + kMetaLast);
  int groups = 0;
  for (int g = 0; g < (p.B + kTokGroup - 1) / kTokGroup; ++g) groups += gfill[g] != 0;
  const uint32_t total = uint32_t(groups * p.n_dstrips);
  bool combined = false;
  for (;;) {
    if (threadIdx.x == 0) {
      int code = -1;
      const uint32_t i = __hip_atomic_fetch_add(p.queue + kQueuePop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (i < total) {
        uint32_t v = 0;
        for (uint32_t n = 0;
             (v = __hip_atomic_load(p.queue + kQueueEnt + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0;
             ++n) {
          if (n >= kSpinLimit) {
            __hip_atomic_store(p.sync + kSyncErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (v) {
          __hip_atomic_store(p.queue + kQueueEnt + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          code = int(v - 1);
        }
      }
      *code_lds = code;
    }
    __syncthreads();
    const int code = *code_lds;
    __syncthreads();
    if (code < 0) break;
    combine_group(p, ds, reinterpret_cast<const uint32_t *>(meta + kMetaFill), code & 0xFF, code >> 8, false);
    combined = true;
  }
  if (combined) MOE_STAMP(9);
  if (threadIdx.x == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's queue accesses are done
    if (__hip_atomic_fetch_add(p.queue + kQueueDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        gridDim.x - 1) {
      __hip_atomic_store(p.queue + kQueuePop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.queue + kQueuePush, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.queue + kQueueDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
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
// one); `first` is the next stage index. Wave 0 meets the grid at the
// barrier (h complete). Meanwhile waves 2 and 3 copy the weights of the next
// kD down stages, all four shares, so those copies overlap the barrier
// without delaying the wait of wave 0 (vmcnt completes in order). Then every
// wave copies its h rows of those stages and waits for all of them.
template <int MTX>
__device__ __forceinline__ void change_to_down(const Params &p, const Stream<MTX> &st, Cursor &prod,
                                               int &issued, int first, unsigned char *stages,
                                               uint32_t rel_base) {
  using S = Shape<2, MTX>;
  constexpr int kS = S::kStages;
  constexpr int kD = kS - 1;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's gate/up stores
  MOE_STAMP(3);
  __syncthreads();
  // h is complete once every workgroup is here (the gate/up epilogues, or
  // the last slice of each tile, formed it).
  if (st.wave == 0) {
    grid_barrier_wave(p.sync, rel_base, 1, true);
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
  MOE_STAMP(4);
  for (int n = 0; n < kD && prod.valid; ++n) {
    st.template issue_a<false>(prod, stages + ((first + n) % kS) * S::kSlot);
    st.advance(prod);
    ++issued;
  }
  wait_barrier<0>();
  MOE_STAMP(5);
}

// The whole bf16 expert FFN in one persistent kernel (one workgroup per CU,
// all resident together):
//   1. gate/up items stream G and U and store slice partial sums;
//   2. h = SiLU(g) * u, formed by the epilogue of a whole-d tile or by the
//      workgroup that completes a tile's last d slice (finish_up); one
//      grid barrier (change_to_down);
//   3. down items stream D with h as the A operand and store rows by token
//      slot; each token's strip of y is formed by the workgroup that
//      completes it (finish_down).
// The first down stages' weights are in flight while the workgroup waits at
// the grid barrier; their A tiles are copied once h is complete.
template <int MTX>
__global__ __launch_bounds__(kThreads, 1) void ffn_kernel(Params p, const UpPlan up,
                                                          const int32_t *__restrict__ n_active,
                                                          const int32_t *__restrict__ active,
                                                          const int32_t *__restrict__ offsets) {
  using S = Shape<2, MTX>;
  constexpr int kS = S::kStages;
  constexpr int kD = kS - 1;  // stages in flight ahead of the one in use
  MOE_STAMP(0);
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kS * S::kSlot + kMetaBytes];
  unsigned char *stages = lds;
  unsigned char *meta = lds + kS * S::kSlot;

  // Routing lists into LDS and the barrier release base. Every load is issued
  // before the first value is used, so that the lists cost one round trip to
  // memory, not one per list, and no load or store sits behind a branch (the
  // compiler would sink the load into it): buffer loads past a list's end
  // return zero, the pair lists are loaded in as few rounds of 256 as cover
  // the call's B*k pairs (the entries past them are never read; issuing the
  // rounds for the largest batch every time put about 0.3 us of load
  // instructions ahead of the first weight copies), and the offsets' last
  // rounds clamp to entry kMaxE, which all their lanes then write with the
  // same value.
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
  int32_t offv[kOffRounds], actv[kActRounds];
#pragma unroll
  for (int r = 0; r < kOffRounds; ++r)
    offv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_off, min(int(threadIdx.x) + r * kThreads, kMaxE) * 4, 0, 0);
#pragma unroll
  for (int r = 0; r < kActRounds; ++r)
    actv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_act, (int(threadIdx.x) + r * kThreads) * 4, 0, 0);
  auto lists = [&](auto rounds_tag) __attribute__((always_inline)) {
    constexpr int R = decltype(rounds_tag)::value;
    int32_t tokv[R], slotv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
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
    for (int r = 0; r < R; ++r) {
      const int i = int(threadIdx.x) + r * kThreads;
      meta[kMetaTok + i] = uint8_t(tokv[r]);
      reinterpret_cast<int16_t *>(meta + kMetaRow)[i] = int16_t(tokv[r] * p.k + slotv[r]);
    }
  };
  if (p.P <= kThreads) lists(std::integral_constant<int, 1>{});
  else if (p.P <= 4 * kThreads) lists(std::integral_constant<int, 4>{});
  else lists(std::integral_constant<int, kPairRounds>{});
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
  MOE_STAMP(1);

  // The gate/up split for this many active experts, chosen on the host
  // (plan_gate_up): stages of kBK rows per d slice, all of d for whole tiles.
  const int up_tiles = nact * p.n_ustrips;
  Split sp;
  if constexpr (MTX < 4) {
    const uint32_t e = (up.e2[nact >> 1] >> (16 * (nact & 1))) & 0xFFFFu;
    sp.slices = int((e >> 8) & 0x7Fu);
    sp.slice_rows = int(e & 0xFFu) * kBK;
    sp.up_whole = sp.slices == 1 ? up_tiles : (e & kUpMixed) ? up_tiles / int(gridDim.x) * int(gridDim.x) : 0;
    // Whole tiles in one round with workgroups to spare: the strips at byte
    // offset 384 mod 512 of each weight row (strips 4q+3 when a row is a
    // multiple of 512 bytes) stream about 20% slower than the others (per-
    // strip stage stamps, on every XCD and in any item order), so their
    // tiles set the end of gate/up. Those tiles are split in two d slices
    // on workgroups that would otherwise wait (Qwen3-30B-shaped B=16
    // oea(4): FFN 34.8 -> 33.6 us; B=8 oea(4) 33.5 -> 31.0; Qwen3-235B-
    // shaped B=1 topk 63.5 -> 57.7).
    sp.slow = 0;
    const int nblk = (p.d + kBK - 1) / kBK;
    const bool strips4 = (p.n_ustrips & 3) == 0 && (p.I * 2) % 512 == 0;
    if (sp.slices == 1 && strips4 && p.slices >= 2 && nblk >= 4 &&
        up_tiles + nact * (p.n_ustrips >> 2) <= int(gridDim.x)) {
      sp.slow = 1;
      sp.slices = 2;
      sp.slice_rows = (nblk + 1) / 2 * kBK;
      sp.up_whole = nact * (p.n_ustrips - (p.n_ustrips >> 2));
    } else if (sp.slices > 1 && sp.up_whole > 0 && strips4) {
      // Mixed plan: the slow strips' tiles last, so that the tiles split in
      // the last round are mostly theirs and the workgroups that take a
      // slice after a whole tile hold the other strips (Qwen3-30B-shaped
      // B=32 oea(4) 59.2 -> 58.0 us, B=16 topk 59.8 -> 58.9).
      sp.slow = 1;
    }
    sp.nfast = sp.slow ? nact * (p.n_ustrips - (p.n_ustrips >> 2)) : sp.up_whole;
  } else {
    // 64-token passes: decided here, by a simpler rule (reading the table,
    // or running plan_split here, slowed this instantiation's stage loop
    // by 2-6%): as many of the planned slices as leave every item a
    // workgroup of its own, else whole d.
    const int nblk = (p.d + kBK - 1) / kBK;
    const int sl = min(p.slices, int(gridDim.x) / max(up_tiles, 1));
    if (sl <= 1 || up_tiles > kMaxTileCounters) {
      sp.slices = 1;
      sp.slice_rows = p.d;
      sp.up_whole = up_tiles;
    } else {
      const int blk = (nblk + sl - 1) / sl;
      sp.slices = (nblk + blk - 1) / blk;
      sp.slice_rows = blk * kBK;
      sp.up_whole = 0;
    }
    sp.slow = 0;
    sp.nfast = sp.up_whole;
  }
  // The down split: as many I slices, up to the planned number (whose
  // partial rows the workspace holds), as leave every down item a workgroup
  // of its own (small active sets), in whole stages.
  {
    const int nbi = (p.I + kBK - 1) / kBK;
    const int ds = max(1, min(p.dslices, int(gridDim.x) / max(nact * p.n_dstrips, 1)));
    const int blk = (nbi + ds - 1) / ds;
    sp.dslices = (nbi + blk - 1) / blk;
    sp.dslice_rows = blk * kBK;
  }

  const Stream<MTX> st(p, sp, lds_addr(meta));
  Cursor cons;
  cons.per_dn = p.n_dstrips * sp.dslices;
  cons.n_up = sp.up_whole + (up_tiles - sp.up_whole) * sp.slices;
  cons.n_items = cons.n_up + nact * cons.per_dn;
  cons.item = blockIdx.x;
  st.decode(cons);
  Cursor prod = cons;

  // Prologue: kD stages in flight (gate/up only: down stages wait for h).
  // `issued` counts the stages issued so far.
  int issued = 0;
  for (int s = 0; s < kD; ++s) {
    if (!prod.valid || !prod.up) break;
    st.issue_up(prod, stages + s * S::kSlot);
    ++issued;
    st.advance(prod);
  }

  Acc acc;
  clear(acc);
  const uint32_t base = lds_addr(stages);
  // One stage of the consumer: stage s must have landed (the stages issued
  // after it may stay in flight, S::kCopies copies per wave each); every wave
  // is then past stage s-1, so its slot takes stage s+kD, whose copies are
  // issued in two halves during the compute of stage s. The gate/up and down
  // phases run in loops of their own (UP), each with only its own code.
  auto stage = [&](int s, auto up_tag) __attribute__((always_inline)) {
    constexpr bool UP = decltype(up_tag)::value;
    const int newer = issued - s - 1;
    switch (newer < kD - 1 ? newer : kD - 1) {
      case 0: wait_barrier<0>(); break;
      case 1: wait_barrier<1 * S::kCopies>(); break;
      case 2: wait_barrier<(kD - 1 >= 2 ? 2 : 0) * S::kCopies>(); break;
      default: wait_barrier<(kD - 1 >= 3 ? 3 : 0) * S::kCopies>(); break;
    }
    MOE_STAGE_STAMP(s, !UP);
    // Gate/up: the producer stops at the first down stage (change_to_down).
    const bool fill = prod.valid && (!UP || prod.up);
    unsigned char *fslot = stages + ((s + kD) % kS) * S::kSlot;
    compute_stage<MTX>(base + uint32_t((s % kS) * S::kSlot), st.trc, st.xrd, st.tp(cons), acc,
                       [&](int half) {
                         if (fill) st.template issue_half<UP>(prod, fslot, half);
                       });
    if (s == 0) MOE_STAMP(2);
    if (fill) {
      ++issued;
      st.advance(prod);
    }
    if (cons.kst == cons.nst - 1) {
      epilogue<MTX, UP>(cons, p, st.meta, st.wave, st.lane, acc);
      clear(acc);
      if constexpr (UP) {
        if (cons.ks >= 0 && (cons.pass + 1) * kMaxTok >= cons.T)
          finish_up(cons, p, sp, reinterpret_cast<int *>(meta + kMetaNLast));
      } else {
        finish_down<(MTX == 4)>(cons, p, sp, meta, st.wave, st.lane);
      }
    }
    st.advance(cons);
  };
  int s = 0;
  for (; cons.valid && cons.up; ++s) stage(s, std::true_type{});
  change_to_down<MTX>(p, st, prod, issued, s, stages, rel_base);
  for (; cons.valid; ++s) stage(s, std::false_type{});
  if constexpr (MTX == 4) drain_combines(p, sp.dslices, meta);
  MOE_STAMP(10);
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

// Per device: compute units and how many workgroups of each instantiation of
// the persistent FFN kernel one CU holds, queried on the first launch on that
// device and cached (several host threads may race to fill an entry; they
// store the same values).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_resident[kMaxDevices][3];

template <int MTX>
constexpr int mtx_index() { return MTX == 1 ? 0 : MTX == 2 ? 1 : 2; }

template <int MTX>
int query_resident_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ffn_kernel<MTX>, kThreads, 0) != hipSuccess) return 0;
  return n;
}

// Compute units of the current device and the workgroups of ffn_kernel<MTX>
// that can be resident on the whole device at once (0 when unknown).
template <int MTX>
void device_limits(int &cus, int &resident) {
  int dev = 0;
  cus = 0;
  resident = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  cus = cached ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      cus = 0;
      return;
    }
    if (cached) g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  int per_cu = cached ? g_resident[dev][mtx_index<MTX>()].load(std::memory_order_relaxed) : 0;
  if (per_cu <= 0) {
    per_cu = query_resident_per_cu<MTX>();
    if (cached && per_cu > 0) g_resident[dev][mtx_index<MTX>()].store(per_cu, std::memory_order_relaxed);
  }
  resident = per_cu * cus;
}

// Gate/up split (plan_split) for every possible active-expert count n (the
// count is only known on the device).
static_assert(kMaxDim / kBK <= 255, "stages per slice fit a byte");
void plan_gate_up(const Params &p, int G, UpPlan &up) {
  for (uint32_t &w : up.e2) w = 0;
  const int nblk = ceil_div(p.d, kBK);
  const int strips = ceil_div(p.I, kStripCols);
  const int planned = p.slices;
  for (int n = 0; n <= p.E; ++n) up.e2[n >> 1] |= plan_split(n * strips, nblk, planned, G) << (16 * (n & 1));
}

// One workgroup per CU at most (grid = min(items, CUs)), so that the whole
// grid is resident together and its grid barriers cannot wait on a
// workgroup that has not started. A device whose CUs cannot hold the grid
// gets hipErrorCooperativeLaunchTooLarge instead of a launch.
template <int MTX>
hipError_t ffn_grid(int items, int &grid) {
  int cus = 0, resident = 0;
  device_limits<MTX>(cus, resident);
  if (cus <= 0) return hipErrorInvalidDevice;
  grid = items < cus ? items : cus;
  return resident < grid ? hipErrorCooperativeLaunchTooLarge : hipSuccess;
}

template <int MTX>
hipError_t launch_ffn(int items, Params &p, const moe_routing_t &r, hipStream_t s) {
  int grid = 0;
  const hipError_t e = ffn_grid<MTX>(items, grid);
  if (e != hipSuccess) return e;
  UpPlan up;
  plan_gate_up(p, grid, up);
  ffn_kernel<MTX><<<grid, kThreads, 0, s>>>(p, up, r.n_active, r.active_experts, r.expert_offsets);
  return hipGetLastError();
}

int ffn_items(int B, int d, int E, int I, int k, const Workspace &plan) {
  const int P = B * k;
  const int max_active = E < P ? E : P;
  return max_active * (ceil_div(I, kStripCols) * plan.up_slices + ceil_div(d, 2 * kStripCols) * plan.dn_slices);
}

}  // namespace

#ifdef MOE_PHASE_STAMPS
uint64_t *g_phase_stamps = nullptr;
#endif

hipError_t expert_ffn_launchable(moe_dtype_t dt, int B, int d, int E, int I, int k, const Workspace &plan) {
  if (dt != MOE_BF16) return hipSuccess;
  const int items = ffn_items(B, d, E, I, k, plan);
  int grid = 0;
  if (B <= 16) return ffn_grid<1>(items, grid);
  if (B <= 32) return ffn_grid<2>(items, grid);
  return ffn_grid<4>(items, grid);
}

hipError_t launch_expert_ffn(const void *x, const void *w_gate, const void *w_up,
                             const void *w_down, moe_dtype_t dt, int B, int d, int E, int I,
                             int k, const moe_routing_t &r, void *y, char *ws,
                             const Workspace &plan, hipStream_t s) {
  const int P = B * k;
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
    p.P = P;
    p.gpart = reinterpret_cast<float *>(ws + plan.up_part);
    p.h = reinterpret_cast<uint16_t *>(ws + plan.h);
    p.part = part;
    p.y = static_cast<uint16_t *>(y);
    p.w = r.topk_w;
    p.pair_token = r.pair_token;
    p.pair_slot = r.pair_slot;
    p.sync = reinterpret_cast<uint32_t *>(ws);
#ifdef MOE_PHASE_STAMPS
    p.stamps = g_phase_stamps;
#endif
    p.grp_cnt = reinterpret_cast<uint32_t *>(ws + kGrpCntOffset);
    p.tile_cnt = reinterpret_cast<uint32_t *>(ws + kTileCntOffset);
    p.queue = reinterpret_cast<uint32_t *>(ws + kQueueOffset);
    p.n_dstrips = ceil_div(d, 2 * kStripCols);
    p.n_ustrips = ceil_div(I, kStripCols);
    p.dslices = plan.dn_slices;
    const int items = ffn_items(B, d, E, I, k, plan);
    // An expert has at most B tokens: A tiles of 16 * MTX rows cover them
    // (experts with more than 64 tokens take several passes).
    if (B <= 16) return launch_ffn<1>(items, p, r, s);
    if (B <= 32) return launch_ffn<2>(items, p, r, s);
    return launch_ffn<4>(items, p, r, s);
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

#ifdef MOE_PHASE_STAMPS
// Measurement library only: where the next bf16 expert FFN launches record
// their phase stamps (device pointer to 256 x 64 uint64, or NULL for none).
extern "C" void moe_phase_stamps(void *stamps) { moe::g_phase_stamps = static_cast<uint64_t *>(stamps); }
#endif
