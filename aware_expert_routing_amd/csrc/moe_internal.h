// Internal declarations shared by the host entry points and the kernel
// translation units of libmoe_decode. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <cmath>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

// ---------------------------------------------------------------- envelope
constexpr int kMaxB = 256;
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;
constexpr int kMaxDim = 16384;

// Router: rows of W_g per partial-sum slice; 16 x 16 logit tiles.
constexpr int kRouterRows = 128;
constexpr int kRouterTile = 16;

// Expert FFN tiling (bf16 path). A work item is one active expert times one
// strip of kStripCols output columns times one slice of the reduction.
constexpr int kStripCols = 64;
constexpr int kUpMaxSlices = 8;     // reduction (d) slices of the gate/up product
constexpr int kUpSliceMin = 512;    // rows per slice before the slice count grows
constexpr int kStageRows = 128;     // weight rows staged in LDS per pipeline stage
constexpr int kDnMaxSlices = 8;     // reduction (I) slices of the down product
// Partial-sum bytes beyond which the slice counts stop growing: gate/up takes
// up to one slice per stage while its partial sums fit kUpPartBudget (else
// one per kUpSliceMin rows of d), down up to one per stage of I while its
// partial rows fit kDnPartBudget.
constexpr size_t kUpPartBudget = size_t(16) << 20;
constexpr size_t kDnPartBudget = size_t(8) << 20;

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Width of the LYNX policy's confidence bins: ln(E / k), rounded to float32
// once on the host so that every kernel compares against the same value.
inline float lynx_bin_width(int E, int k) { return float(std::log(double(E) / double(k))); }

// The first kCounterBytes of every workspace hold counters at fixed offsets
// (the same for every size of call, so that calls of different sizes may
// share a workspace): the expert FFN's grid-barrier words (first 384 bytes),
// the fused router + selection counter, the router's per-tile counters (up
// to 256 tiles), the FFN's per-(16-token group, 128-column strip of d)
// counters, each of those on a 128-byte line of its own, the FFN's
// per-gate/up-tile slice counters (atomics on one line are served one after
// another) and the FFN's combine queue. All are zero before the workspace's
// first use. Every call leaves the counters at zero; the barrier's release
// word only grows. No other step writes them.
constexpr size_t kSyncBytes = 2048;
constexpr size_t kSyncErrOffset = 256;         // FFN: non-zero once a grid-barrier wait gave up
static_assert(kSyncErrOffset + 4 <= MOE_WS_STATUS_BYTES, "status word inside the status bytes");
constexpr size_t kRouteSelectCntOffset = 384;  // fused router + selection: tiles done
constexpr size_t kRouterCntOffset = 512;
constexpr int kTokGroup = 16;                      // tokens per combine group
constexpr int kTokGroups = kMaxB / kTokGroup;      // groups at B = kMaxB
constexpr int kCntStride = 32;                     // uint32 words between group counters
constexpr size_t kGrpCntOffset = kSyncBytes;       // [kMaxDim / 128 strips][kTokGroups] x 128 B
// FFN, sliced gate/up path: per gate/up tile (active expert, 64-column strip
// of I), the d slices counted so far, each on a 64-byte piece of a line.
// Tiles past kMaxTileCounters take the whole-d path (no counter needed).
constexpr int kMaxTileCounters = 4096;
constexpr int kTileCntStride = 16;                 // uint32 words between tile counters
constexpr size_t kTileCntOffset =
    kGrpCntOffset + size_t(kMaxDim / (2 * kStripCols)) * kTokGroups * kCntStride * 4;
// FFN, batches of more than 32 tokens: the combine queue. The pop index, the
// push index and the count of workgroups done, each on a 128-byte line, then
// one word per (128-column strip of d, token group) combine in push order
// (0 until pushed).
constexpr size_t kQueueOffset = kTileCntOffset + size_t(kMaxTileCounters) * kTileCntStride * 4;
constexpr int kMaxCombines = (kMaxDim / (2 * kStripCols)) * kTokGroups;
constexpr size_t kCounterBytes = kQueueOffset + 3 * 128 + size_t(kMaxCombines) * 4;

// Workspace carve-up. Every segment starts on a 256-byte boundary.
struct Workspace {
  size_t router_part;  // float [tiles][router_slices][16 x 16] partial logit tiles
  size_t up_part;      // float [up_slices][2][B*k][I]   (gate, up partial sums)
  size_t h;            // bf16 or float [B*k][I]
  size_t down_part;    // float [dn_slices][B*k][d], one row per (I slice, expert-token pair)
  size_t pair_of_slot; // int32 [B*k]: pair index of token slot t*k+j
  size_t total;
  int router_slices;
  int up_slices;
  int up_slice_rows;
  int dn_slices;       // most I slices of the down product (the kernel may use fewer)
};

inline Workspace plan_workspace(int B, int d, int E, int I, int k, moe_dtype_t dt) {
  Workspace w{};
  w.router_slices = ceil_div(d, kRouterRows);
  const size_t router_tiles = size_t(ceil_div(E, kRouterTile)) * ceil_div(B, kRouterTile);
  const size_t P = size_t(B) * size_t(k);
  // Partial-sum regions: at least the minimum slice count's bytes, at least
  // the budget when more slices fit it, so that a region never shrinks as B
  // grows (a workspace sized for the largest call serves every smaller one).
  const size_t up_slice_bytes = 2 * P * size_t(I) * sizeof(float);
  int s_min = ceil_div(d, kUpSliceMin);
  if (s_min > kUpMaxSlices) s_min = kUpMaxSlices;
  int s_max = ceil_div(d, kStageRows);
  if (s_max > kUpMaxSlices) s_max = kUpMaxSlices;
  size_t up_bytes = size_t(s_max) * up_slice_bytes;
  if (up_bytes > kUpPartBudget) up_bytes = kUpPartBudget;
  if (up_bytes < size_t(s_min) * up_slice_bytes) up_bytes = size_t(s_min) * up_slice_bytes;
  int slices = int(up_bytes / up_slice_bytes);
  if (slices > s_max) slices = s_max;
  if (slices < s_min) slices = s_min;
  int rows = ceil_div(d, slices);
  rows = ceil_div(rows, kStageRows) * kStageRows;
  w.up_slices = ceil_div(d, rows);
  w.up_slice_rows = rows;
  const size_t dn_slice_bytes = P * size_t(d) * sizeof(float);
  int ds_max = ceil_div(I, kStageRows);
  if (ds_max > kDnMaxSlices) ds_max = kDnMaxSlices;
  if (dt != MOE_BF16) ds_max = 1;
  size_t dn_bytes = size_t(ds_max) * dn_slice_bytes;
  if (dn_bytes > kDnPartBudget) dn_bytes = kDnPartBudget;
  if (dn_bytes < dn_slice_bytes) dn_bytes = dn_slice_bytes;
  w.dn_slices = int(dn_bytes / dn_slice_bytes);
  if (w.dn_slices > ds_max) w.dn_slices = ds_max;
  const size_t esz = (dt == MOE_BF16) ? 2 : 4;
  size_t off = kCounterBytes;
  w.router_part = off;
  off = align256(off + router_tiles * w.router_slices * kRouterTile * kRouterTile * sizeof(float));
  w.up_part = off;
  if (dt == MOE_BF16) off = align256(off + up_bytes);
  w.h = off;
  off = align256(off + P * I * esz);
  w.down_part = off;
  off = align256(off + dn_bytes);
  w.pair_of_slot = off;
  off = align256(off + P * sizeof(int32_t));
  w.total = off;
  return w;
}

// Size of the file-scope scratch array of moe_layer_decode_static (per
// device); calls whose workspace plan exceeds it are refused.
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;

// ------------------------------------------------------------- launchers
// Each launcher enqueues on `s` and returns hipGetLastError().

// logits = x W_g + bias in one launch; part holds the partial tiles, cnt the
// per-tile counters (zero before, zero after).
hipError_t launch_router(const void *x, const void *w_g, const float *bias, moe_dtype_t dt, int B,
                         int d, int E, float *part, uint32_t *cnt, float *logits, hipStream_t s);

// Selection on float32 logits[B,E].
hipError_t launch_select(const float *logits, int B, int E, moe_policy_t p,
                         const moe_routing_t &r, hipStream_t s);

// bf16 router and selection in one launch; part holds the slices' partial
// logit tiles, cnt is a counter word (zero before, zero after).
hipError_t launch_route_select(const void *x, const void *w_g, const float *bias, int B, int d,
                               int E, float *logits, float *part, uint32_t *cnt, moe_policy_t p,
                               const moe_routing_t &r, hipStream_t s);

// Read-only scan of `bytes` (a multiple of 16) at src by kReadStreamBlocks
// workgroups; out[b] receives workgroup b's XOR of the words it read.
constexpr int kReadStreamBlocks = 1024;
hipError_t launch_read_stream(const void *src, size_t bytes, uint32_t *out, hipStream_t s);

// Whether launch_expert_ffn can run these sizes on the current device (bf16:
// its persistent grid fits the device's resident-workgroup limit). Launches
// nothing; hipErrorCooperativeLaunchTooLarge when the grid cannot be resident.
hipError_t expert_ffn_launchable(moe_dtype_t dt, int B, int d, int E, int I, int k, const Workspace &plan);

hipError_t launch_expert_ffn(const void *x, const void *w_gate, const void *w_up,
                             const void *w_down, moe_dtype_t dt, int B, int d, int E, int I,
                             int k, const moe_routing_t &r, void *y, char *ws,
                             const Workspace &plan, hipStream_t s);

// moe_layer_decode_static's scratch: the current device's address of the
// file-scope array (looked up once per device), and a launch that zeroes its
// counter region on stream s.
hipError_t static_scratch_address(char **out);
hipError_t clear_scratch_counters(char *ptr, hipStream_t s);

}  // namespace moe
