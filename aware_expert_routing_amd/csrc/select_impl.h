#pragma once
#include <type_traits>
// Ranking, batch re-route, gate weights and compaction, in one workgroup
// (device function select_block; used by select.hip and route_select.hip).
//
//   ranking   "Router Caching and Optimization", "Analyzing Router Inference
//             Cost", steps 2-3: softmax and top-k; experts are ranked by
//             logit (softmax is increasing), ties to the lower index, and
//             -0.0 ranks equal to +0.0.
//   OEA(k0)   "Opportunistic Expert Activation", abstract: tokens keep their
//             top-k0; S = union over the batch; each token then fills up to k
//             slots with its best experts inside S.
//   BUDGET(m) "XShare", abstract: maximise the total gating score. The batch
//             mass of expert e is the sum over tokens of softmax(logits_t)[e];
//             the m largest masses (ties to the lower index) form the set.
//   GREEDY(m) "XShare", abstract (greedy solution): the set grows one expert
//             at a time by the largest gain in retained mass
//             F(S) = sum_t (sum of t's k largest probabilities inside S); the
//             gain of e is sum_t max(0, p_t[e] - thr_t), thr_t being t's k-th
//             largest probability in S (0 while t has fewer than k there);
//             ties to the lower index.
//   HIER(m, m_r, g)  "XShare", summary and abstract (hierarchical selection
//             for speculative batches; the steps are the reading taken here):
//             the batch keeps the BUDGET(m) set; request r (tokens r*g ..
//             r*g+g-1) keeps the m_r experts of that set with the largest
//             mass summed over its own tokens, in token order (ties to the
//             lower index); its tokens rank inside that request set.
//   LYNX(m)   "Lynx", Technical Summary 2.1 and 2.2 (the constants are
//             the reading taken here): the gap between a token's rank-0 logit
//             and each of its top-k logits (float32) falls into one of k
//             bins of width bin_w = ln(E/k) (bin = number of i in 1..k-1 with
//             gap >= i * bin_w, float32 products); an expert scores
//             2^(k-1-bin) per (token, rank < k) naming it (integer sums, so
//             the order of the atomics does not matter); the critical set
//             holds every rank-0 expert plus the best-scored other named
//             experts (ties to the lower index) up to max(m, |rank-0 set|);
//             tokens take their first k experts inside it.
//   weights   softmax over each token's selected logits.
//   compact   "Lynx", Technical Summary 2.2: the batch activates one
//             consolidated expert set; this kernel lists it (ascending) and
//             the tokens of each active expert (ascending).
//
// Work split: the batch step couples all tokens, so one workgroup of 16 waves
// does everything. Wave w owns tokens w, w+16, ...; lane l owns experts l,
// l+64, ... (NV = ceil(E/64) of them). A token's experts are ranked by
// repeated wave-wide maxima of order-preserving 32-bit keys; among equal keys
// the lowest expert index is read off the ballots of "key == max" (scalar
// work). Key 0 is no finite logit's key and marks "not a candidate".
//
// Results stay in LDS until the last phase: per (token, slot) the expert and
// weight, per expert a bitmask of its tokens. The position of token t in
// expert e's list is then the number of lower tokens in that bitmask, so the
// pair lists are written by all threads at once.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxTokPerWave = kMaxB / kWaves;  // token slots per wave at B = 256
constexpr int kWords = kMaxE / 32;           // words of an expert bitmask
constexpr int kTokWords = kMaxB / 32;        // words of a token bitmask
constexpr int kGreedyTable = 8192;           // greedy: largest B * E held in LDS
constexpr int kGreedyWaves = 4;              // greedy: waves running the rounds
constexpr int kSpinLimit = 1 << 22;          // greedy: polls of the arrival count

// Total order on float32 as unsigned integers; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t ord_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ord_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Wave-wide reductions with DPP lane moves (gfx9 encodings): quad_perm
// [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror, then row_bcast:15
// into rows 1 and 3 and row_bcast:31 into rows 2 and 3. After the six steps
// lane 63 holds the result over all 64 lanes; readlane makes it uniform.
constexpr int kDppQuadX1 = 0xB1;
constexpr int kDppQuadX2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

// Lanes that a step does not write keep `old`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), CTRL, ROWS, 0xF, false));
}

// The same six steps with the lane move folded into the arithmetic (one
// v_max_u32_dpp / v_add_f32_dpp per step: dst = op(moved v, v); rows that a
// step does not write keep v). Two wait states precede every step, since each
// reads through DPP the register the previous instruction wrote.
#define MOE_DPP_STEPS(OP)                                                        \
  "s_nop 1\n" OP " %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n" \
  "s_nop 1\n" OP " %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n" \
  "s_nop 1\n" OP " %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"     \
  "s_nop 1\n" OP " %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n"          \
  "s_nop 1\n" OP " %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n"        \
  "s_nop 1\n" OP " %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n"        \
  "s_nop 1\n"

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  asm volatile(MOE_DPP_STEPS("v_max_u32_dpp") : "+v"(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the wave in a fixed tree; every lane gets the lane-63 result, so
// the value is uniform and reproducible from run to run. (Lane 63 takes part
// in every step, so rows left out of a step do not affect it.)
__device__ __forceinline__ float wave_sum(float v) {
  asm volatile(MOE_DPP_STEPS("v_add_f32_dpp") : "+v"(v));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Inclusive prefix sum over the wave: within each row of 16 lanes by
// shifts of 1, 2, 4 and 8 lanes (lanes shifted in from outside the row add
// 0), then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// then rows 0-1's total into rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ __forceinline__ int scan_step(int v) {
  return v + int(dpp<CTRL, ROWS>(0u, uint32_t(v)));
}

__device__ __forceinline__ int wave_scan_incl(int v) {
  v = scan_step<0x111, 0xF>(v);  // row_shr:1
  v = scan_step<0x112, 0xF>(v);  // row_shr:2
  v = scan_step<0x114, 0xF>(v);  // row_shr:4
  v = scan_step<0x118, 0xF>(v);  // row_shr:8
  v = scan_step<kDppBcast15, 0xA>(v);
  v = scan_step<kDppBcast31, 0xC>(v);
  return v;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float fmax_step(float v) {
  return fmaxf(v, __uint_as_float(dpp<CTRL, ROWS>(__float_as_uint(v), __float_as_uint(v))));
}

__device__ __forceinline__ float wave_maxf(float v) {
  v = fmax_step<kDppQuadX1, 0xF>(v);
  v = fmax_step<kDppQuadX2, 0xF>(v);
  v = fmax_step<kDppHalfMirror, 0xF>(v);
  v = fmax_step<kDppMirror, 0xF>(v);
  v = fmax_step<kDppBcast15, 0xA>(v);
  v = fmax_step<kDppBcast31, 0xC>(v);
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float fmin_step(float v) {
  return fminf(v, __uint_as_float(dpp<CTRL, ROWS>(__float_as_uint(v), __float_as_uint(v))));
}

__device__ __forceinline__ float wave_minf(float v) {
  v = fmin_step<kDppQuadX1, 0xF>(v);
  v = fmin_step<kDppQuadX2, 0xF>(v);
  v = fmin_step<kDppHalfMirror, 0xF>(v);
  v = fmin_step<kDppMirror, 0xF>(v);
  v = fmin_step<kDppBcast15, 0xA>(v);
  v = fmin_step<kDppBcast31, 0xC>(v);
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Up to `rounds` rounds of wave-wide argmax over the keys (expert lane+64v
// holds key[v]). Lane r receives the r-th winner's expert and key; `top` is
// the first winner's key. Returns the number of winners.
template <int NV>
__device__ __forceinline__ int wave_rank(uint32_t (&key)[NV], int rounds, int base, int lane,
                                         int &my_e, uint32_t &my_key, uint32_t &top) {
  int n = 0;
  for (int r = 0; r < rounds; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int v = 1; v < NV; ++v) best = key[v] > best ? key[v] : best;
    best = wave_max_u32(best);
    if (best == 0) break;
    int e = 0;
#pragma unroll
    for (int v = NV - 1; v >= 0; --v) {  // the lowest index holding `best` wins
      const unsigned long long b = __ballot(key[v] == best);
      if (b) e = 64 * v + __builtin_ctzll(b);
    }
    if (lane == base + r) {
      my_e = e;
      my_key = best;
    }
    if (base + r == 0) top = best;
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if (lane + 64 * v == e) key[v] = 0;
    ++n;
  }
  return n;
}

__device__ __forceinline__ bool bit_of(const uint32_t *mask, int e) { return (mask[e >> 5] >> (e & 31)) & 1u; }

// Descending rank of every key among key[0..E) (ties to the lower index),
// added into rank[] (zero before; read after a barrier): rank[e] counts the
// e2 with key[e2] > key[e], or key[e2] == key[e] and e2 < e. The E x E
// comparisons are spread over the whole workgroup: thread (part, e) compares
// key[e] with a quarter of the keys, 16 bytes per LDS read, and adds its
// count with one LDS atomic (integer, so the sum does not depend on order).
// key must be 16-byte aligned with room for kMaxE entries.
__device__ __forceinline__ void rank_keys_desc(const uint32_t *key, int E, int *rank) {
  constexpr int kParts = kThreads / kMaxE;
  static_assert(kParts * kMaxE == kThreads && kMaxE % (4 * kParts) == 0, "rank split");
  const int e = threadIdx.x % kMaxE, part = threadIdx.x / kMaxE;
  if (e >= E) return;
  const uint32_t ke = key[e];
  const int span = (((E + kParts - 1) / kParts) + 3) & ~3;
  const int lo = part * span, hi = min(E, lo + span);
  int r = 0;
  for (int e0 = lo; e0 < hi; e0 += 4) {
    const uint4 o = *reinterpret_cast<const uint4 *>(key + e0);
    r += e0 < hi && ((o.x > ke) || (o.x == ke && e0 < e));
    r += e0 + 1 < hi && ((o.y > ke) || (o.y == ke && e0 + 1 < e));
    r += e0 + 2 < hi && ((o.z > ke) || (o.z == ke && e0 + 2 < e));
    r += e0 + 3 < hi && ((o.w > ke) || (o.w == ke && e0 + 3 < e));
  }
  if (r) atomicAdd(&rank[e], r);
}

// Source of the float32 logits: logit(t, e) with 0 <= t < B, 0 <= e < E;
// gather(L, B, wave, lane), which fills L[ti][v] with logit(min(wave + 16ti,
// B - 1), min(lane + 64v, E - 1)) for every slot, issuing the loads of
// several slots before the first is used; and emit(t, e, v), called once for
// every (t, e) with the value read. Logits stored in memory: device-scope
// loads (another workgroup of the same kernel may have stored them); nothing
// to emit.
struct StoredLogits {
  const float *p;
  int E;
  __device__ __forceinline__ float operator()(int t, int e) const {
    return __hip_atomic_load(const_cast<float *>(p) + t * E + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  template <int TPW, int NV>
  __device__ __forceinline__ void gather(float (&L)[TPW][NV], int B, int wave, int lane) const {
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
      for (int v = 0; v < NV; ++v) L[ti][v] = (*this)(min(wave + kWaves * ti, B - 1), min(lane + 64 * v, E - 1));
  }
  __device__ __forceinline__ void emit(int, int, float) const {}
};

// The whole selection, run by one workgroup of kThreads threads, on the
// logits of `src`. TPW token slots per wave (B <= 16 * TPW): the per-token
// phases are unrolled over the slots, so a small TPW keeps the code small.
template <int NV, int TPW, class Src>
__device__ __forceinline__ void select_block(
    const Src &src, int B, int E, int kind, int k, int k0, int m, int g, float bin_w,
    int32_t *__restrict__ topk_ids, float *__restrict__ topk_w, int32_t *__restrict__ n_active,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ pair_token, int32_t *__restrict__ pair_slot,
    float *__restrict__ batch_mass) {
  __shared__ uint32_t allowed[kWords];
  __shared__ uint32_t req_allowed[kMaxB][kWords];  // HIER: each request's set
  __shared__ uint32_t etok[kMaxE][kTokWords];  // bit t of etok[e]: token t routes to e
  __shared__ int16_t sel_id[kMaxB][kMaxK];
  __shared__ float sel_w[kMaxB][kMaxK];
  __shared__ float psum[kWaves][kMaxE];
  __shared__ __attribute__((aligned(16))) float mass[kMaxE];
  __shared__ int krank[kMaxE];  // BUDGET, HIER, LYNX: rank of each expert's key
  __shared__ int acnt[kMaxE];
  __shared__ int apos[kMaxE];
  __shared__ int aoff[kMaxE];
  __shared__ int s_n, s_total;
  __shared__ __attribute__((aligned(16))) uint32_t lscore[kMaxE];  // LYNX: expert scores
  __shared__ uint32_t lrank0[kWords];  // LYNX: rank-0 experts of the batch
  __shared__ unsigned long long g_best[2];  // GREEDY: each round's best (gain, expert)
  __shared__ float gP[TPW <= 4 ? kGreedyTable : 1];  // GREEDY: probabilities [B][E]
  __shared__ int g_arrive;                  // GREEDY: arrivals of the four greedy waves
  __shared__ int g_first[kMaxK];       // GREEDY: the first rounds' picks in order

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int i = tid; i < kWords; i += kThreads) {
    uint32_t full = 0;
    if (kind == MOE_POLICY_TOPK) {
      const int lo = i * 32;
      const int nb = min(32, max(0, E - lo));
      full = nb == 32 ? 0xFFFFFFFFu : ((1u << nb) - 1u);
    }
    allowed[i] = full;
  }
  for (int i = tid; i < kMaxE * kTokWords; i += kThreads) etok[i / kTokWords][i % kTokWords] = 0;
  if (kind == MOE_POLICY_LYNX) {
    for (int i = tid; i < kMaxE; i += kThreads) lscore[i] = 0;
    for (int i = tid; i < kWords; i += kThreads) lrank0[i] = 0;
  }
  for (int i = tid; i < kMaxE; i += kThreads) krank[i] = 0;
  if (kind == MOE_POLICY_HIER)
    for (int i = tid; i < ((B + g - 1) / g) * kWords; i += kThreads) req_allowed[i / kWords][i % kWords] = 0;

  // Phase 1: logits into registers. Indices are clamped so that every read
  // is in bounds; values outside [B, E) are never used as candidates.
  float L[TPW][NV];
  src.template gather<TPW, NV>(L, B, wave, lane);
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    const int t = wave + kWaves * ti;
    if (t < B)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if (lane + 64 * v < E) src.emit(t, lane + 64 * v, L[ti][v]);
  }
  __syncthreads();

  // Phase 2: the policy's batch step. OEA keeps each token's top-k0 picks
  // (lane j holds pick j): they are also the first k0 picks of phase 3, since
  // they are the token's largest logits and all of them are allowed.
  int pick_e[TPW], pick_n[TPW];
  uint32_t pick_key[TPW], pick_top[TPW], picked[TPW];  // bit v of picked: candidate lane+64v taken
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    pick_e[ti] = 0;
    pick_n[ti] = 0;
    pick_key[ti] = 0;
    pick_top[ti] = 0;
    picked[ti] = 0;
  }
  if (kind == MOE_POLICY_OEA) {
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int t = wave + kWaves * ti;
      if (t < B) {
        uint32_t key[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) key[v] = (lane + 64 * v < E) ? ord_bits(L[ti][v]) : 0u;
        uint32_t cand = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) cand |= uint32_t(key[v] != 0) << v;
        const int n = wave_rank<NV>(key, k0, 0, lane, pick_e[ti], pick_key[ti], pick_top[ti]);
#pragma unroll
        for (int v = 0; v < NV; ++v) picked[ti] |= uint32_t(((cand >> v) & 1u) && key[v] == 0) << v;
        pick_n[ti] = n;
        if (lane < n) atomicOr(&allowed[pick_e[ti] >> 5], 1u << (pick_e[ti] & 31));
      }
    }
  } else if (kind == MOE_POLICY_BUDGET || kind == MOE_POLICY_HIER) {
    // Per-token softmax over all E experts, then column sums over the batch
    // in a fixed order (token slot ti outer, wave inner).
    float macc = 0.0f;  // thread tid < E accumulates expert tid
    const int rounds = (B + kWaves - 1) / kWaves;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      if (ti < rounds) {  // block-uniform: every wave reaches the same barriers
        const int t = wave + kWaves * ti;
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (lane + 64 * v < E) mx = fmaxf(mx, L[ti][v]);
        mx = wave_maxf(mx);
        float sm = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (lane + 64 * v < E) sm += expf(L[ti][v] - mx);
        sm = wave_sum(sm);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int e = lane + 64 * v;
          if (e < E) psum[wave][e] = (t < B) ? expf(L[ti][v] - mx) / sm : 0.0f;
        }
        __syncthreads();
        if (tid < E) {
          for (int w = 0; w < kWaves; ++w) macc += psum[w][tid];
        }
        __syncthreads();
      }
    }
    if (tid < E) mass[tid] = macc;
    __syncthreads();
    // Masses are sums of non-negative terms (never -0.0), so their bit
    // patterns order like the values.
    rank_keys_desc(reinterpret_cast<const uint32_t *>(mass), E, krank);
    __syncthreads();
    if (tid < E && krank[tid] < m) atomicOr(&allowed[tid >> 5], 1u << (tid & 31));
    if (kind == MOE_POLICY_HIER) {
      // Request level: wave w takes requests w, w+16, ...; a request's mass
      // is summed over its tokens in order (each token's softmax recomputed
      // from the logits by the same expression as above), then ranked inside
      // the batch set with the same wave ranking as the tokens (k0 = m_r).
      __syncthreads();  // the batch set is complete
      const int R = (B + g - 1) / g;
      for (int r = wave; r < R; r += kWaves) {
        float Mr[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) Mr[v] = 0.0f;
        const int t1 = min(B, r * g + g);
        for (int t0 = r * g; t0 < t1; t0 += 4) {
          // Four token rows per round trip (rows past the request are
          // clamped loads, never used).
          float lv[4][NV];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < NV; ++v)
              lv[q][v] = src(min(t0 + q, t1 - 1), min(lane + 64 * v, E - 1));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (t0 + q < t1) {  // wave-uniform; tokens in order
              float mx = -INFINITY;
#pragma unroll
              for (int v = 0; v < NV; ++v)
                if (lane + 64 * v < E) mx = fmaxf(mx, lv[q][v]);
              mx = wave_maxf(mx);
              float sm = 0.0f;
#pragma unroll
              for (int v = 0; v < NV; ++v)
                if (lane + 64 * v < E) sm += expf(lv[q][v] - mx);
              sm = wave_sum(sm);
#pragma unroll
              for (int v = 0; v < NV; ++v)
                if (lane + 64 * v < E) Mr[v] += expf(lv[q][v] - mx) / sm;
            }
          }
        }
        uint32_t key[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int e = lane + 64 * v;
          key[v] = (e < E && bit_of(allowed, e)) ? ord_bits(Mr[v]) : 0u;
        }
        int pe = 0;
        uint32_t pk = 0, ptop = 0;
        const int n = wave_rank<NV>(key, k0, 0, lane, pe, pk, ptop);
        if (lane < n) atomicOr(&req_allowed[r][pe >> 5], 1u << (pe & 31));
      }
    }
  } else if (kind == MOE_POLICY_LYNX) {
    // Confidence bins of each token's top-k and the experts' scores.
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int t = wave + kWaves * ti;
      if (t < B) {
        uint32_t key[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) key[v] = (lane + 64 * v < E) ? ord_bits(L[ti][v]) : 0u;
        uint32_t cand = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) cand |= uint32_t(key[v] != 0) << v;
        // The token's top-k are kept (lane j holds pick j): the leading ones
        // that fall inside the critical set start phase 3.
        const int n = wave_rank<NV>(key, k, 0, lane, pick_e[ti], pick_key[ti], pick_top[ti]);
#pragma unroll
        for (int v = 0; v < NV; ++v) picked[ti] |= uint32_t(((cand >> v) & 1u) && key[v] == 0) << v;
        pick_n[ti] = n;
        if (lane < n) {
          const float gap = from_ord_bits(pick_top[ti]) - from_ord_bits(pick_key[ti]);
          int bin = 0;
          for (int i = 1; i < k; ++i) bin += gap >= float(i) * bin_w;
          const int e = pick_e[ti];
          atomicAdd(&lscore[e], 1u << (k - 1 - bin));
          if (lane == 0) atomicOr(&lrank0[e >> 5], 1u << (e & 31));
        }
      }
    }
    __syncthreads();
    // Critical set: the rank-0 experts, then the other named experts (score
    // > 0) by score descending, ties to the lower index. Rank-0 experts drop
    // out of the ranking (score set to 0, as for experts nobody named).
    const bool rank0 = tid < E && bit_of(lrank0, tid);
    if (rank0) lscore[tid] = 0;
    __syncthreads();
    rank_keys_desc(lscore, E, krank);
    __syncthreads();
    if (tid < E) {
      int n0 = 0;
      for (int w = 0; w < kWords; ++w) n0 += __popc(lrank0[w]);
      // A named expert's score is at least 1, so zero keys (rank-0 and
      // unnamed experts) never rank above one.
      const bool keep = rank0 || (lscore[tid] > 0 && krank[tid] < m - n0);
      if (keep) atomicOr(&allowed[tid >> 5], 1u << (tid & 31));
    }
  } else if (kind == MOE_POLICY_GREEDY) {
    // Each token's probabilities, computed once from the logits.
    float pr[TPW][NV];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int t = wave + kWaves * ti;
#pragma unroll
      for (int v = 0; v < NV; ++v) pr[ti][v] = 0.0f;
      if (t < B) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (lane + 64 * v < E) mx = fmaxf(mx, L[ti][v]);
        mx = wave_maxf(mx);
        float sm = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (lane + 64 * v < E) sm += expf(L[ti][v] - mx);
        sm = wave_sum(sm);
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (lane + 64 * v < E) pr[ti][v] = expf(L[ti][v] - mx) / sm;
      }
    }
    // Up to 64 tokens with the probability table in LDS: four waves run the
    // rounds (the others wait at the barrier that ends this phase). Greedy
    // wave gw holds the probabilities of tokens gw, gw + 4, gw + 8, ... in
    // registers and the k largest of each inside S in one 16-lane row of a
    // list register (descending in lanes 0..k-1, 0 where S holds fewer than
    // k: the probabilities are >= 0, so lane k-1 is the threshold). Each
    // round it adds its tokens' terms in order, meets the other three on an
    // LDS arrival count (no workgroup barrier inside the rounds), adds the
    // four partial gains in wave order and takes the same argmax as the
    // others. While S holds fewer than k experts every threshold is 0, so
    // the first min(k, m) rounds reuse the first round's gains.
    const bool table = TPW <= 4 && B * E <= kGreedyTable;  // block-uniform
    if constexpr (TPW <= 4) {
      if (table) {
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) {
          const int t = wave + kWaves * ti;
          if (t < B)
#pragma unroll
            for (int v = 0; v < NV; ++v)
              if (lane + 64 * v < E) gP[t * E + lane + 64 * v] = pr[ti][v];
        }
        if (tid == 0) g_arrive = 0;
        __syncthreads();
        if (wave < kGreedyWaves) {
          constexpr int kGT = kGreedyWaves * TPW;  // token slots of a greedy wave
          const int gw = wave;
          float P[kGT][NV];
#pragma unroll
          for (int i = 0; i < kGT; ++i) {
            const int t = min(gw + kGreedyWaves * i, B - 1);
#pragma unroll
            for (int v = 0; v < NV; ++v) P[i][v] = gP[t * E + min(lane + 64 * v, E - 1)];
          }
          float lst[TPW];  // list register q: row r holds token slot 4q + r
          float thr[kGT];
#pragma unroll
          for (int q = 0; q < TPW; ++q) lst[q] = 0.0f;
#pragma unroll
          for (int i = 0; i < kGT; ++i) thr[i] = 0.0f;
          uint32_t key[NV], tk = 0;  // bit v of tk: expert lane + 64v is in S
#pragma unroll
          for (int v = 0; v < NV; ++v) key[v] = 0;
          float *part = &psum[0][0];  // [2][kGreedyWaves][kMaxE], alternating
          int rr = 0;                 // exchanges so far
          const int kk = min(k, m);
          for (int r = 0; r < m; ++r) {
            if (r == 0 || r >= kk) {
              float g[NV];
#pragma unroll
              for (int v = 0; v < NV; ++v) g[v] = 0.0f;
#pragma unroll
              for (int i = 0; i < kGT; ++i)
                if (gw + kGreedyWaves * i < B)
#pragma unroll
                  for (int v = 0; v < NV; ++v) g[v] += fmaxf(0.0f, P[i][v] - thr[i]);
              float *mine = part + ((rr & 1) * kGreedyWaves + gw) * kMaxE;
#pragma unroll
              for (int v = 0; v < NV; ++v)
                if (lane + 64 * v < E) mine[lane + 64 * v] = g[v];
              // Arrive after this wave's stores; wait for the other three
              // (bounded: the four waves never wait on anything else).
              if (lane == 0) __hip_atomic_fetch_add(&g_arrive, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
              const int target = kGreedyWaves * (rr + 1);
              for (int it = 0; it < kSpinLimit; ++it)
                if (__hip_atomic_load(&g_arrive, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
              const float *all = part + (rr & 1) * kGreedyWaves * kMaxE;
#pragma unroll
              for (int v = 0; v < NV; ++v) {
                const int e = min(lane + 64 * v, E - 1);
                float gain = all[e];
#pragma unroll
                for (int w = 1; w < kGreedyWaves; ++w) gain += all[w * kMaxE + e];
                key[v] = lane + 64 * v < E ? ord_bits(gain) : 0u;
              }
              ++rr;
            }
            uint32_t best = 0;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const uint32_t kv = ((tk >> v) & 1u) ? 0u : key[v];
              best = kv > best ? kv : best;
            }
            best = wave_max_u32(best);
            if (best == 0) continue;  // no candidate left (m <= E: never)
            int e = 0;
#pragma unroll
            for (int v = NV - 1; v >= 0; --v) {  // the lowest index holding `best` wins
              const unsigned long long b = __ballot(!((tk >> v) & 1u) && key[v] == best);
              if (b) e = 64 * v + __builtin_ctzll(b);
            }
            if ((e & 63) == lane) tk |= 1u << (e >> 6);
            // Each token inserts its probability of e; a value not above the
            // k-th largest falls past lane k-1 and changes nothing.
#pragma unroll
            for (int q = 0; q < TPW; ++q) {
              if (gw + kGreedyWaves * 4 * q < B) {
                const int t = min(gw + kGreedyWaves * (4 * q + (lane >> 4)), B - 1);
                const float pe = gP[t * E + e];
                const float cur = lst[q];
                const float prev = __uint_as_float(dpp<0x111, 0xF>(__float_as_uint(INFINITY), __float_as_uint(cur)));
                lst[q] = cur >= pe ? cur : (prev >= pe ? pe : prev);
#pragma unroll
                for (int row = 0; row < 4; ++row)
                  thr[4 * q + row] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lst[q]), 16 * row + k - 1));
              }
            }
          }
          if (wave == 0) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
              if ((tk >> v) & 1u) atomicOr(&allowed[(lane + 64 * v) >> 5], 1u << ((lane + 64 * v) & 31));
          }
        }
      }
    }
    if (!table) {
      // Token slot ti's k largest probabilities inside S, in descending order
      // in lanes 0..k-1 (-1: no value yet), and its threshold thr (the k-th
      // largest, 0 while S holds fewer than k experts). Wave-uniform thr.
      float lst[TPW], thr[TPW];
#pragma unroll
      for (int ti = 0; ti < TPW; ++ti) {
        lst[ti] = -1.0f;
        thr[ti] = 0.0f;
      }
      // Each token slot inserts its probability of expert e into its list; a
      // value not above the k-th largest falls past lane k-1 and changes
      // nothing.
      auto insert = [&](int e) {
        const int ve = e >> 6, le = e & 63;
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) {
          if (wave + kWaves * ti < B) {
            float x = 0.0f;
#pragma unroll
            for (int v = 0; v < NV; ++v)
              if (v == ve) x = pr[ti][v];
            const float pe = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), le));
            // Lane j-1's entry (lane 0: +inf), row_shr:1 inside lanes 0..15.
            const float prev = __uint_as_float(dpp<0x111, 0xF>(__float_as_uint(INFINITY), __float_as_uint(lst[ti])));
            const float cur = lst[ti];
            lst[ti] = cur >= pe ? cur : (prev >= pe ? pe : prev);
            thr[ti] = fmaxf(0.0f, __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lst[ti]), k - 1)));
          }
        }
      };
      bool taken = false;  // thread tid < E: expert tid is in S
      // While S holds fewer than k experts every threshold is 0, so the
      // first min(k, m) rounds all see the first round's gains: they take
      // that round's largest gains in order (ties to the lower index) at once.
      const int kk = min(k, m);
      // Round r's best (gain, expert) key, larger gain first, then the lower
      // index (complemented in the low word); the two slots alternate.
      if (tid == 0) g_best[0] = g_best[1] = 0ull;
      for (int r = 0; r < m; ++r) {
        // Gains over this wave's token slots in order, then over the waves in
        // order (by the threads tid < E, one expert each; waves without tokens
        // add 0).
        {
          float g[NV];
#pragma unroll
          for (int v = 0; v < NV; ++v) g[v] = 0.0f;
#pragma unroll
          for (int ti = 0; ti < TPW; ++ti)
            if (wave + kWaves * ti < B)
#pragma unroll
              for (int v = 0; v < NV; ++v) g[v] += fmaxf(0.0f, pr[ti][v] - thr[ti]);
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const int e = lane + 64 * v;
            if (e < E) psum[wave][e] = g[v];
          }
        }
        __syncthreads();
        uint32_t key = 0;  // thread tid < E: expert tid's gain (0: not a candidate)
        if (tid < E && !taken) {
          // All rows loaded before the first add (one LDS round trip).
          float part[kWaves];
#pragma unroll
          for (int w = 0; w < kWaves; ++w) part[w] = psum[w][tid];
          // Pairwise, in a fixed tree.
#pragma unroll
          for (int h = 1; h < kWaves; h *= 2)
#pragma unroll
            for (int w = 0; w < kWaves; w += 2 * h) part[w] += part[w + h];
          key = ord_bits(part[0]);
        }
        if (r == 0 && kk > 1) {
          uint32_t *gkey = lscore;  // free outside LYNX
          if (tid < E) gkey[tid] = key;
          __syncthreads();
          rank_keys_desc(gkey, E, krank);
          __syncthreads();
          if (tid < E && krank[tid] < kk) {
            taken = true;
            g_first[krank[tid]] = tid;
          }
          __syncthreads();
          for (int j = 0; j < min(kk, E); ++j) insert(g_first[j]);
          r = kk - 1;
          continue;
        }
        if (wave * 64 < E) {
          const uint32_t best = wave_max_u32(key);
          const unsigned long long b = __ballot(key == best && key != 0);
          // A uniform value: one lane's atomic, no wave reduction around it.
          const uint32_t lo = __builtin_amdgcn_readfirstlane(~uint32_t(wave * 64 + __builtin_ctzll(b)));
          if (lane == 0 && b) atomicMax(&g_best[r & 1], (uint64_t(best) << 32) | lo);
        }
        // The other slot was last read before this round's first barrier.
        if (tid == 0) g_best[(r + 1) & 1] = 0ull;
        __syncthreads();
        const uint64_t bp = g_best[r & 1];
        if (bp == 0) break;  // block-uniform: no expert left
        const int e = int(~uint32_t(bp));
        if (tid == e) taken = true;
        insert(e);
      }
      if (tid < E && taken) atomicOr(&allowed[tid >> 5], 1u << (tid & 31));
    }
  }
  __syncthreads();

  // Phase 3: each token takes its best experts inside the allowed set.
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    const int t = wave + kWaves * ti;
    if (t < B) {
      uint32_t key[NV];
      const uint32_t *mask = kind == MOE_POLICY_HIER ? req_allowed[t / g] : allowed;
      if (kind == MOE_POLICY_LYNX) {
        // Only the leading picks inside the critical set are the first picks
        // of the masked order; the later ones become candidates again.
        const unsigned long long in =
            __ballot(lane < pick_n[ti] && bit_of(mask, pick_e[ti]));
        const int pre = int(__builtin_ctzll(~in));
        for (int r = pre; r < pick_n[ti]; ++r) {
          const int er = __builtin_amdgcn_readlane(pick_e[ti], r);
#pragma unroll
          for (int v = 0; v < NV; ++v)
            if (lane + 64 * v == er) picked[ti] &= ~(1u << v);
        }
        pick_n[ti] = pre;
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int e = lane + 64 * v;
        key[v] = (e < E && bit_of(mask, e) && !((picked[ti] >> v) & 1u)) ? ord_bits(L[ti][v]) : 0u;
      }
      // Continue after the picks phase 2 already made (none unless OEA).
      int e = pick_e[ti];
      uint32_t kv = pick_key[ti], top = pick_top[ti];
      const int n = pick_n[ti] + wave_rank<NV>(key, k - pick_n[ti], pick_n[ti], lane, e, kv, top);
      const float ex = lane < n ? expf(from_ord_bits(kv) - from_ord_bits(top)) : 0.0f;
      const float tot = wave_sum(ex);
      if (lane < k) {
        sel_id[t][lane] = int16_t(lane < n ? e : -1);
        sel_w[t][lane] = lane < n ? ex / tot : 0.0f;
      }
      if (lane < n) atomicOr(&etok[e][t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();

  // Phase 4: wave 0 counts each expert's tokens and scans the counts; lane l
  // owns experts l*NV .. l*NV+NV-1 so that the scan runs in expert order.
  if (wave == 0) {
    const int nw = (B + 31) >> 5;
    int c[NV], a[NV];
    int lc = 0, la = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = lane * NV + v;
      int cv = 0;
      if (e < E)
        for (int w = 0; w < nw; ++w) cv += __popc(etok[e][w]);
      c[v] = cv;
      a[v] = cv > 0;
      lc += c[v];
      la += a[v];
    }
    const int ic = wave_scan_incl(lc), ia = wave_scan_incl(la);  // inclusive scans over lanes
    int pc = ic - lc, pa = ia - la;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = lane * NV + v;
      if (e < E) {
        acnt[e] = c[v];
        aoff[e] = pc;
        apos[e] = pa;
      }
      pc += c[v];
      pa += a[v];
    }
    if (lane == 63) {
      s_total = ic;
      s_n = ia;
    }
  }
  __syncthreads();

  // Phase 5: every output, written once, by all threads.
  const int nact = s_n, total = s_total, P = B * k;
  if (tid < E && acnt[tid] > 0) {
    active_experts[apos[tid]] = tid;
    expert_offsets[apos[tid]] = aoff[tid];
  }
  if (tid < E && batch_mass) batch_mass[tid] = mass[tid];
  for (int i = nact + tid; i < E; i += kThreads) active_experts[i] = -1;
  for (int i = nact + tid; i <= E; i += kThreads) expert_offsets[i] = total;
  for (int i = tid; i < P; i += kThreads) {
    const int t = i / k, j = i - t * k;
    const int e = sel_id[t][j];
    topk_ids[i] = e;
    topk_w[i] = sel_w[t][j];
    if (e >= 0) {
      const uint32_t *row = etok[e];
      int pos = aoff[e];
      for (int w = 0; w < (t >> 5); ++w) pos += __popc(row[w]);
      pos += __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
      pair_token[pos] = t;
      pair_slot[pos] = j;
    }
  }
  for (int i = total + tid; i < P; i += kThreads) {
    pair_token[i] = -1;
    pair_slot[i] = -1;
  }
  if (tid == 0) n_active[0] = nact;
}

// Calls f(NV tag, TPW tag) with the compile-time expert and token-slot
// counts that cover E and B.
template <typename F>
__host__ void dispatch_select_shape(int B, int E, F &&f) {
  auto by_b = [&](auto nv) {
    if (B <= kWaves) f(nv, std::integral_constant<int, 1>{});
    else if (B <= 4 * kWaves) f(nv, std::integral_constant<int, 4>{});
    else f(nv, std::integral_constant<int, kMaxTokPerWave>{});
  };
  if (E <= 64) by_b(std::integral_constant<int, 1>{});
  else if (E <= 128) by_b(std::integral_constant<int, 2>{});
  else by_b(std::integral_constant<int, 4>{});
}

}  // namespace
}  // namespace moe
