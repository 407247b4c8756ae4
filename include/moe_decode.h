/*
 * moe_decode.h -- C ABI of the decode-time MoE layer with batch-aware expert
 * selection, for AMD Instinct MI355X (gfx950).
 *
 * The layer (one decode step, B tokens):
 *   1. router:    logits[t,e] = sum_i x[t,i] * W_g[i,e] + bias[e]
 *                 ("Router Caching and Optimization", section "Analyzing
 *                 Router Inference Cost", step 1, linear projection).
 *   2. ranking:   each token orders the experts by logit, highest first, ties
 *                 to the lower index; softmax and top-k follow from it (same
 *                 section, steps 2 and 3).
 *   3. re-route:  a batch-level policy shrinks the set of experts the batch
 *                 activates:
 *                   TOPK       standard per-token top-k;
 *                   OEA(k0)    each token keeps its top-k0; S is the union of
 *                              these over the batch; each token then takes its
 *                              highest-ranked experts inside S, up to k
 *                              ("Opportunistic Expert Activation", abstract);
 *                   BUDGET(m)  the m experts with the largest softmax mass
 *                              summed over the batch form the allowed set; each
 *                              token takes its top min(k,m) inside it ("XShare",
 *                              abstract: maximise the total gating score);
 *                   GREEDY(m)  the allowed set grows greedily, one expert at a
 *                              time, by the largest gain in the batch's
 *                              retained top-k softmax mass (ties to the lower
 *                              index), m experts in all; each token takes its
 *                              top min(k,m) inside it ("XShare", abstract).
 *                   HIER(m, m_r, g)  speculative batches: tokens form requests
 *                              of g consecutive tokens (one request's
 *                              drafts); the batch keeps the BUDGET(m) set;
 *                              each request keeps the m_r experts of it with
 *                              the largest softmax mass summed over the
 *                              request's tokens (ties to the lower index);
 *                              each token takes its top min(k, m_r) inside
 *                              its request's set ("XShare", summary and
 *                              abstract: hierarchical selection for
 *                              speculative decoding; the reading taken here).
 *                   LYNX(m)    confidence-gated remap ("Lynx", Technical
 *                              Summary 2.1 and 2.2; constants are the
 *                              reading taken here): the gap between a token's
 *                              rank-0 logit and each of its top-k logits is
 *                              binned into k bins of width ln(E/k) (float32);
 *                              an expert scores 2^(k-1-bin) per (token, rank
 *                              < k) naming it; the critical set holds every
 *                              token's rank-0 expert plus the best-scored
 *                              other experts named by some top-k (ties to the
 *                              lower index), max(m, |rank-0 set|) in all, as
 *                              far as there are such experts; each token
 *                              takes its first k experts inside it, so every
 *                              token keeps exactly k.
 *   4. weights:   gate weights are the softmax over each token's selected
 *                 logits (renormalised); empty slots weigh 0.
 *   5. compaction: the ascending list of active experts and, per active
 *                 expert, its tokens in ascending order ("Lynx", Technical
 *                 Summary 2.2: the batch activates one consolidated set).
 *   6. expert FFN: y[t] = sum_j w[t,j] * (SiLU(x_t G_e) * (x_t U_e)) D_e with
 *                 e the expert in slot j, SiLU(z) = z / (1 + exp(-z)); only the
 *                 active experts' weights are read from HBM ("Lynx", Technical
 *                 Summary 1: latency follows the number of distinct experts).
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers to contiguous row-major arrays,
 *     owned by the caller. The library keeps no pointer after it returns.
 *   - x, w_g, w_gate, w_up, w_down and y share one element type, `dt`
 *     (MOE_F32: float; MOE_BF16: bfloat16 bit patterns, uint16). Logits,
 *     bias, gate weights and batch masses are always float32; ids int32.
 *   - Layouts: x[B,d], w_g[d,E], bias[E], w_gate[E,d,I], w_up[E,d,I],
 *     w_down[E,I,d], logits[B,E], y[B,d].
 *   - `stream` is a hipStream_t (NULL: the default stream). Calls only
 *     enqueue work and return; results are valid once the stream reaches
 *     them. No call allocates, frees or synchronises, so calls can be
 *     captured into a HIP graph.
 *   - Every argument is checked on the host before any HIP call; a failed
 *     check returns an error code and enqueues nothing. No C++ exception
 *     crosses this interface. The only state kept between calls is, per
 *     device, its compute-unit count and the expert FFN's resident-workgroup
 *     limit, queried on the first call on that device and cached thread-
 *     safely. Calls are safe from several host threads on different streams
 *     with different workspaces.
 *   - Non-finite inputs give unspecified results.
 *
 * Supported envelope (else MOE_ERR_UNSUPPORTED): 1 <= B <= 256,
 * 1 <= E <= 256, 1 <= k <= 16, 8 <= d <= 16384 and 8 <= I <= 16384 with d and
 * I multiples of 8. Pointers to x, w_g, w_gate, w_up, w_down and y must be
 * 16-byte aligned (else MOE_ERR_INVALID_ARG).
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null/misaligned pointer, k > E, k0 or m out of range, ... */
  MOE_ERR_UNSUPPORTED = 2, /* sizes outside the supported envelope above              */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than required  */
  MOE_ERR_HIP = 4,         /* a kernel launch failed (hipGetLastError)                 */
  MOE_ERR_RESIDENCY = 5,   /* the bf16 expert FFN's workgroups (one per compute unit)
                              cannot all be resident on this device: nothing launched */
  MOE_ERR_SYNC_TIMEOUT = 6, /* from moe_workspace_check: a grid-wide wait of the bf16
                              expert FFN gave up in some call since the workspace was
                              zero-filled; those calls' outputs are unspecified        */
  MOE_ERR_SCRATCH = 7,     /* moe_layer_decode_static: the sizes need more scratch than
                              its static array holds (MOE_STATIC_SCRATCH_BYTES)        */
  MOE_STATUS_FORCE_32BIT = 0x7FFFFFFF /* not a status: makes every int32 value a valid
                              moe_status_t, so that unknown codes are well defined  */
} moe_status_t;

/* Bytes at the start of a workspace that moe_workspace_check reads. */
#define MOE_WS_STATUS_BYTES 512

/* Size of the static scratch of moe_layer_decode_static, per device. */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_DTYPE_FORCE_32BIT = 0x7FFFFFFF /* not a dtype: every int32 value is a valid
                                        moe_dtype_t (others are rejected)      */
} moe_dtype_t;

typedef enum {
  MOE_POLICY_TOPK = 0,   /* k experts per token (k <= E)                         */
  MOE_POLICY_OEA = 1,    /* 1 <= k0 <= k; tokens get min(k, |S|) experts         */
  MOE_POLICY_BUDGET = 2, /* 1 <= m <= E; tokens get min(k, m) experts            */
  MOE_POLICY_GREEDY = 3, /* 1 <= m <= E; tokens get min(k, m) experts            */
  MOE_POLICY_HIER = 4,   /* 1 <= k0 = m_r <= m <= E, g >= 1; tokens get
                            min(k, m_r) experts                                  */
  MOE_POLICY_LYNX = 5    /* k <= m <= E; tokens get exactly k experts            */
} moe_policy_kind_t;

/* Selection policy. k0 is read by OEA (its k0) and HIER (the request budget
 * m_r); m by BUDGET, GREEDY, HIER (the batch budget) and LYNX (the size of
 * the critical set); g only by HIER (tokens per request: token t belongs to
 * request t / g). */
typedef struct {
  int32_t kind; /* moe_policy_kind_t */
  int32_t k;
  int32_t k0;
  int32_t m;
  int32_t g;
} moe_policy_t;

/* Routing outputs (device pointers, caller-owned, written in full by every
 * call that produces them; sizes use the call's B, E and k). */
typedef struct {
  int32_t *topk_ids;       /* [B,k] slot order = logit desc, index asc; -1 = empty */
  float *topk_w;           /* [B,k] renormalised gate weight; 0 for empty slots    */
  int32_t *n_active;       /* [1]   experts that receive >= 1 token                */
  int32_t *active_experts; /* [E]   ascending expert ids, then -1                  */
  int32_t *expert_offsets; /* [E+1] CSR offsets over the active list; entries past
                                    n_active repeat the number of pairs           */
  int32_t *pair_token;     /* [B*k] token of each (expert, token) pair, tokens
                                    ascending within an expert; then -1           */
  int32_t *pair_slot;      /* [B*k] slot j of that pair in topk_ids; then -1        */
  float *batch_mass;       /* [E]   BUDGET and HIER: sum over tokens of
                                    softmax(logits_t); may be NULL for the other
                                    policies, which leave it alone               */
} moe_routing_t;

/* Bytes of workspace the calls below need for these sizes (256-byte aligned
 * base required). Returns 0 when the sizes are outside the envelope.
 *
 * The workspace must be zero-filled once, before its first use (e.g.
 * hipMemset after allocation); afterwards the caller must not write it. Its
 * first bytes hold the synchronisation words of the bf16 expert FFN (grid
 * barrier, a counter per output column strip and 16-token group, a counter
 * per gate/up tile when the gate/up product is split over d, and, above 32
 * tokens, a queue of (strip, group) combines that every workgroup drains),
 * which every call leaves ready for the next one. The same workspace may serve
 * consecutive calls on one stream; calls that may overlap need separate
 * workspaces. The bf16 expert FFN runs one workgroup per compute unit and
 * needs all of them resident together: a device whose compute units cannot
 * hold its grid gets MOE_ERR_RESIDENCY at launch; do not run it next to
 * another kernel that waits on work of its own. If a grid-wide wait
 * nevertheless exceeds its bound (about a million polls), the kernel records
 * it in the workspace's status bytes, which stay set until the workspace is
 * zero-filled again, and finishes with unspecified outputs (it never hangs);
 * moe_workspace_check reports it. */
size_t moe_workspace_bytes(int B, int d, int E, int I, int k, moe_dtype_t dt);

/* Reads the status of a workspace: `status_host` is a HOST copy of the first
 * MOE_WS_STATUS_BYTES bytes of the workspace (e.g. hipMemcpy after the
 * stream has reached the calls to check), `bytes` its size. Returns
 * MOE_ERR_SYNC_TIMEOUT if a grid-wide wait of the bf16 expert FFN gave up in
 * any call since the workspace was last zero-filled, MOE_OK otherwise, and
 * MOE_ERR_INVALID_ARG for a null pointer or bytes < MOE_WS_STATUS_BYTES.
 * Host-only: makes no HIP call. Callers that cannot afford the copy after
 * every call may check once after a batch of calls. */
moe_status_t moe_workspace_check(const void *status_host, size_t bytes);

/* Step 1 only: logits[B,E] (float32) = x W_g + bias. bias may be NULL (zero).
 * Uses the workspace (after the synchronisation words) for per-slice partial
 * sums; it needs at least moe_workspace_bytes(B, d, E, 8, 1, dt) bytes. */
moe_status_t moe_route(const void *x, const void *w_g, const float *bias, moe_dtype_t dt,
                       int B, int d, int E, float *logits, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Steps 2-5 on given float32 logits[B,E]: writes every field of *out.
 * BUDGET requires out->batch_mass. Needs no workspace. */
moe_status_t moe_select(const float *logits, int B, int E, moe_policy_t policy,
                        const moe_routing_t *out, void *stream);

/* Step 6 for routing produced by moe_select (same B, E, k): y[B,d] in dt.
 * Reads only the weights of the first *n_active experts of the active list. */
moe_status_t moe_expert_ffn(const void *x, const void *w_gate, const void *w_up,
                            const void *w_down, moe_dtype_t dt, int B, int d, int E, int I,
                            int k, const moe_routing_t *routing, void *y, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Steps 1-6: the whole decode MoE layer. logits[B,E] receives the router
 * output; *routing receives the selection as moe_select writes it. */
moe_status_t moe_layer_decode(const void *x, const void *w_g, const float *bias,
                              const void *w_gate, const void *w_up, const void *w_down,
                              moe_dtype_t dt, int B, int d, int E, int I, moe_policy_t policy,
                              float *logits, const moe_routing_t *routing, void *y,
                              void *workspace, size_t workspace_bytes, void *stream);

/* moe_layer_decode without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid allocation). Same arguments, outputs, checks and results as
 * moe_layer_decode; the scratch memory is a static device array of
 * MOE_STATIC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends (looked up on the first call on a device).
 *   - Sizes whose moe_workspace_bytes exceeds MOE_STATIC_SCRATCH_BYTES get
 *     MOE_ERR_SCRATCH and enqueue nothing (at d = 2048, E = 128, I = 768,
 *     k = 8 every B up to 64 fits).
 *   - Every call on a device shares that device's array: calls that may
 *     overlap in time on one device (different streams, no ordering between
 *     them) race and give unspecified results. Calls ordered on one stream
 *     are fine.
 *   - Each call first zeroes the array's counters (one small kernel), so a
 *     call cut short cannot affect the next one; a grid-wide wait that gives
 *     up is not reported (moe_layer_decode with a workspace reports it).
 *   - Allocates nothing: no hipMalloc, hipFree or allocating library call. */
moe_status_t moe_layer_decode_static(const void *x, const void *w_g, const float *bias,
                                     const void *w_gate, const void *w_up, const void *w_down,
                                     moe_dtype_t dt, int B, int d, int E, int I, moe_policy_t policy,
                                     float *logits, const moe_routing_t *routing, void *y,
                                     void *stream);

/* Static description of a status code. Never NULL. */
const char *moe_status_string(moe_status_t status);

/* Measurement utility, not a step of the layer: a read-only scan of `bytes`
 * bytes at device pointer `src` (16-byte aligned, bytes a positive multiple
 * of 16) by 1024 workgroups, each reading one contiguous block with 16-byte
 * loads; out[1024] (device, uint32) receives each workgroup's XOR of the
 * words it read. Its rate is the plain-streaming read ceiling of the GPU that
 * the expert FFN's rate is compared with. MOE_ERR_INVALID_ARG on a null or
 * misaligned pointer or a bad size; nothing else is checked or written. */
moe_status_t moe_read_stream(const void *src, size_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
