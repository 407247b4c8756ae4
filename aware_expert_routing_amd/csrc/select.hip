// Ranking, batch re-route, gate weights and compaction, in one workgroup.
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
//   weights   softmax over each token's selected logits.
//   compact   "Lynx", Technical Summary 2.2: the batch activates one
//             consolidated expert set; this kernel lists it (ascending) and
//             the tokens of each active expert (ascending).
//
// Work split: the batch step couples all tokens, so one workgroup of 16 waves
// does everything. Wave w owns tokens w, w+16, ...; each lane owns experts
// lane, lane+64, ... A token's experts are ranked by repeated wave-wide
// maximum of 64-bit keys (orderable logit bits << 32 | ~expert): the largest
// key is the largest logit, and among equal logits the lowest index. Key 0
// never occurs for a finite logit, so it marks "no candidate".
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kNV = kMaxE / 64;             // experts per lane
constexpr int kTokPerWave = kMaxB / kWaves;  // tokens per wave
constexpr int kWords = kMaxE / 32;           // words of an expert bitmask

// Total order on float32 as unsigned integers; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t ord_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ord_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float v, int e) {
  return (uint64_t(ord_bits(v)) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(e));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor(uint32_t(v), off);
    const uint32_t hi = __shfl_xor(uint32_t(v >> 32), off);
    const uint64_t o = (uint64_t(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Butterfly sums: partner lanes add the same two values (commutative), so
// every lane ends with the identical, run-to-run reproducible result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Up to `rounds` rounds of wave-wide argmax over the candidate keys. Lane r
// receives the r-th winner. Returns the number of winners.
__device__ __forceinline__ int wave_rank(uint64_t (&key)[kNV], int rounds, int lane, int &my_id,
                                float &my_val, float &first_val) {
  int n = 0;
  for (int r = 0; r < rounds; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int v = 1; v < kNV; ++v) best = key[v] > best ? key[v] : best;
    best = wave_max_u64(best);
    if (best == 0) break;
    const int e = int(0xFFFFFFFFu - uint32_t(best));
    const float val = from_ord_bits(uint32_t(best >> 32));
    if (lane == r) {
      my_id = e;
      my_val = val;
    }
    if (r == 0) first_val = val;
#pragma unroll
    for (int v = 0; v < kNV; ++v)
      if (lane + 64 * v == e) key[v] = 0;
    ++n;
  }
  return n;
}

__device__ __forceinline__ bool bit_of(const uint32_t *mask, int e) { return (mask[e >> 5] >> (e & 31)) & 1u; }

__global__ __launch_bounds__(kThreads) void select_kernel(
    const float *__restrict__ logits, int B, int E, int kind, int k, int k0, int m,
    int32_t *__restrict__ topk_ids, float *__restrict__ topk_w, int32_t *__restrict__ n_active,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ pair_token, int32_t *__restrict__ pair_slot,
    float *__restrict__ batch_mass) {
  __shared__ uint32_t allowed[kWords];
  __shared__ uint32_t tokmask[kMaxB][kWords];
  __shared__ int16_t sel_ids[kMaxB][kMaxK];
  __shared__ float psum[kWaves][kMaxE];
  __shared__ float mass[kMaxE];
  __shared__ int cnt[kMaxE];
  __shared__ int apos[kMaxE];
  __shared__ int aoff[kMaxE];
  __shared__ int s_n, s_total;

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
  for (int i = tid; i < B * kWords; i += kThreads) tokmask[i / kWords][i % kWords] = 0;
  for (int i = tid; i < kMaxE; i += kThreads) cnt[i] = 0;

  __syncthreads();

  float L[kTokPerWave][kNV];
#pragma unroll
  for (int ti = 0; ti < kTokPerWave; ++ti) {
    const int t = wave + kWaves * ti;
#pragma unroll
    for (int v = 0; v < kNV; ++v) {
      const int e = lane + 64 * v;
      L[ti][v] = (t < B && e < E) ? logits[t * E + e] : 0.0f;
    }
  }

  // Phase 2: the policy's batch step.
  if (kind == MOE_POLICY_OEA) {
#pragma unroll
    for (int ti = 0; ti < kTokPerWave; ++ti) {
      const int t = wave + kWaves * ti;
      if (t < B) {
        uint64_t key[kNV];
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
          const int e = lane + 64 * v;
          key[v] = e < E ? make_key(L[ti][v], e) : 0;
        }
        int id = -1;
        float val = 0.0f, first = 0.0f;
        const int n = wave_rank(key, k0, lane, id, val, first);
        if (lane < n) atomicOr(&allowed[id >> 5], 1u << (id & 31));
      }
    }
  } else if (kind == MOE_POLICY_BUDGET) {
    // Per-token softmax over all E experts, then column sums over the batch
    // in a fixed order (token slot ti outer, wave inner).
    float macc = 0.0f;  // thread tid < E accumulates expert tid
    const int rounds = (B + kWaves - 1) / kWaves;
#pragma unroll
    for (int ti = 0; ti < kTokPerWave; ++ti) {
      if (ti < rounds) {  // block-uniform: every wave reaches the same barriers
        const int t = wave + kWaves * ti;
        float mx = -INFINITY;
  #pragma unroll
        for (int v = 0; v < kNV; ++v)
          if (lane + 64 * v < E) mx = fmaxf(mx, L[ti][v]);
        mx = wave_maxf(mx);
        float sm = 0.0f;
  #pragma unroll
        for (int v = 0; v < kNV; ++v)
          if (lane + 64 * v < E) sm += expf(L[ti][v] - mx);
        sm = wave_sum(sm);
  #pragma unroll
        for (int v = 0; v < kNV; ++v) {
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
    if (tid < E) {
      mass[tid] = macc;
      if (batch_mass) batch_mass[tid] = macc;
    }
    __syncthreads();
    if (tid < E) {
      int rank = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const float o = mass[e2];
        rank += (o > macc) || (o == macc && e2 < tid);
      }
      if (rank < m) atomicOr(&allowed[tid >> 5], 1u << (tid & 31));
    }
  }
  __syncthreads();

  // Phase 3: each token takes its best experts inside the allowed set.
#pragma unroll
  for (int ti = 0; ti < kTokPerWave; ++ti) {
    const int t = wave + kWaves * ti;
    if (t < B) {
      uint64_t key[kNV];
  #pragma unroll
      for (int v = 0; v < kNV; ++v) {
        const int e = lane + 64 * v;
        key[v] = (e < E && bit_of(allowed, e)) ? make_key(L[ti][v], e) : 0;
      }
      int id = -1;
      float val = 0.0f, first = 0.0f;
      const int n = wave_rank(key, k, lane, id, val, first);
      const float ex = lane < n ? expf(val - first) : 0.0f;
      const float tot = wave_sum(ex);
      if (lane < k) {
        topk_ids[t * k + lane] = lane < n ? id : -1;
        topk_w[t * k + lane] = lane < n ? ex / tot : 0.0f;
        sel_ids[t][lane] = int16_t(lane < n ? id : -1);
      }
      if (lane < n) {
        atomicOr(&tokmask[t][id >> 5], 1u << (id & 31));
        atomicAdd(&cnt[id], 1);
      }
    }
  }
  __syncthreads();

  // Phase 4: compaction. Wave 0 scans the per-expert counts.
  if (wave == 0) {
    int c[kNV], a[kNV];
    int lc = 0, la = 0;
#pragma unroll
    for (int v = 0; v < kNV; ++v) {
      const int e = lane * kNV + v;
      c[v] = (e < E) ? cnt[e] : 0;
      a[v] = c[v] > 0;
      lc += c[v];
      la += a[v];
    }
    int ic = lc, ia = la;  // inclusive scans over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oc = __shfl_up(ic, off);
      const int oa = __shfl_up(ia, off);
      if (lane >= off) {
        ic += oc;
        ia += oa;
      }
    }
    int pc = ic - lc, pa = ia - la;
#pragma unroll
    for (int v = 0; v < kNV; ++v) {
      const int e = lane * kNV + v;
      if (e < E) {
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

  const int nact = s_n, total = s_total;
  if (tid < E && cnt[tid] > 0) {
    const int e = tid;
    const int ap = apos[e];
    int c = aoff[e];
    active_experts[ap] = e;
    expert_offsets[ap] = c;
    for (int t = 0; t < B; ++t) {
      if (!bit_of(tokmask[t], e)) continue;
      int j = 0;
      while (sel_ids[t][j] != e) ++j;
      pair_token[c] = t;
      pair_slot[c] = j;
      ++c;
    }
  }
  for (int i = nact + tid; i < E; i += kThreads) active_experts[i] = -1;
  for (int i = nact + tid; i <= E; i += kThreads) expert_offsets[i] = total;
  for (int i = total + tid; i < B * k; i += kThreads) {
    pair_token[i] = -1;
    pair_slot[i] = -1;
  }
  if (tid == 0) n_active[0] = nact;
}

}  // namespace

hipError_t launch_select(const float *logits, int B, int E, moe_policy_t p,
                         const moe_routing_t &r, hipStream_t s) {
  select_kernel<<<1, kThreads, 0, s>>>(logits, B, E, p.kind, p.k, p.k0, p.m,
                                       r.topk_ids, r.topk_w, r.n_active, r.active_experts,
                                       r.expert_offsets, r.pair_token, r.pair_slot, r.batch_mass);
  return hipGetLastError();
}

}  // namespace moe
