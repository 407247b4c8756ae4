"""CPU oracle for the decode-time MoE layer with batch-aware expert selection.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. It shares no code with the HIP path (no
kernels, headers, helpers, tables or pre/post-processing) and imports nothing
from it. It is deliberately plain and slow: numpy, float64 arithmetic, each
step written out in the order the pages describe.

Sources (web pages on the subject; cited by title and section):
  [Router]  "Router Caching and Optimization", section "Analyzing Router
            Inference Cost": linear projection h = x W_g, softmax, top-k; and
            the router-cache example, which ranks by softmax probability.
  [OEA]     "Opportunistic Expert Activation: Batch-Aware Expert Routing for
            Faster Decode Without Retraining", abstract and lay summary: each
            token first keeps its most important experts, then piggybacks on
            experts already loaded for other tokens of the batch.
  [XShare]  "XShare: Collaborative in-Batch Expert Sharing for Faster MoE
            Inference", summary and abstract: batch-aware selection as a
            modular optimisation, maximising the total gating score of the
            selected experts.
  [Lynx]    "Lynx: Enabling Efficient MoE Inference through Dynamic
            Batch-Aware Expert Selection", Technical Summary section 1
            (latency follows the number of distinct experts the batch loads)
            and section 2.2 (the batch activates a consolidated expert set).

Readings where the pages are silent (each is stated where it is used):
  R1  Per-token order: experts sorted by float32 logit descending, ties to
      the lower expert index; -0.0 equals +0.0. Ranking by logit equals
      ranking by probability (softmax is strictly increasing) and avoids
      ties that rounding of exp would create.
  R2  Decisions are taken on float32 values (the precision the kernels
      compute in): logits are rounded to float32 before ranking and the
      budget masses are rounded to float32 before ranking.
  R3  Gate weights are the softmax restricted to the selected experts
      (renormalised), for every policy, so oea(k0 = k) equals top-k.
  R4  oea(k0): S = union over tokens of each token's top-k0; token t takes
      the first min(k, |S|) experts of its own order that lie in S.
  R5  budget(m): per-token softmax over all E experts, summed over the batch
      in token order; the m experts with the largest sum (ties to the lower
      index) form the allowed set; token t takes the first min(k, m)
      experts of its own order inside it.
  R6  SwiGLU expert: y = (SiLU(x G) * (x U)) D with SiLU(z) = z / (1 + e^-z),
      no biases; G, U are [d, I] and D is [I, d] per expert.
  R7  Empty slots (a token with fewer than k experts) carry id -1, weight 0.
  R8  hier(m, m_r, g) for speculative batches ([XShare] summary and
      abstract name a hierarchical, correlation-aware selection for
      speculative decoding without giving its steps): tokens come in
      requests of g consecutive tokens (the drafts of one request). The batch
      keeps the budget(m) set S_b; each request r then keeps the m_r experts
      of S_b with the largest softmax mass summed over its own tokens (in
      token order, ranked as float32, ties to the lower index): S_r; each of
      its tokens takes the first min(k, m_r) experts of its own order inside
      S_r. Both levels maximise the total gating score under their budget,
      the modular objective of [XShare].
  R9  lynx(m), a confidence-gated remap ([Lynx] section 2.1 "Token
      Confidence" and "Expert Rank Hierarchy", section 2.2 "Confidence
      Analyzer", "Adaptive Expert Scorer", "Expert Remapper"; the page gives
      no formulas, so every constant below is the reading taken here):
      * confidence of token t's rank-j expert (j < k) is the logit gap
        delta = L[t, rank 0] - L[t, rank j] (float32 subtraction);
      * AffinityBinning: k bins of width w = ln(E / k) (the inverse sparsity
        ratio N/k on a logit scale), rounded to float32; the bin is the
        number of i in 1..k-1 with delta >= float32(i) * w (float32
        product), i.e. min(k - 1, floor(delta / w));
      * the expert scorer adds 2^(k - 1 - bin) for every (token, rank < k)
        pair naming the expert (an integer: confident pairs weigh
        exponentially more);
      * the critical set C holds every token's rank-0 expert (rank 0 is
        kept), then the other experts named by some token's top-k, by score
        descending (ties to the lower index), until |C| = max(m, |R0|) or
        no such expert is left;
      * the remapper gives token t the first k experts of its own order
        inside C. With k <= m every token keeps exactly k experts, as the
        page requires.

Parity status of each function is listed in its docstring ("pinned by ...").
"""
from __future__ import annotations

import math

import numpy as np

POLICY_TOPK = "topk"
POLICY_OEA = "oea"
POLICY_BUDGET = "budget"
POLICY_GREEDY = "greedy"
POLICY_HIER = "hier"
POLICY_LYNX = "lynx"


# ---------------------------------------------------------------- precision

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening to float64. ``dtype`` "bf16" means ``a`` holds uint16
    bfloat16 bit patterns; "f32" means float32 values."""
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 inputs are float32")
        return a.astype(np.float64)
    raise ValueError(dtype)


def _finite(*arrs):
    for a in arrs:
        if a is not None and not np.all(np.isfinite(a)):
            raise ValueError("inputs must be finite")


# -------------------------------------------------------------------- router

def router_logits(x, w_g, bias, dtype: str) -> np.ndarray:
    """Router linear projection, [Router] "Analyzing Router Inference Cost",
    step 1: h = x W_g (per token), plus a per-expert bias (the workloads'
    skewed router bias; None means zero). float64 result [B, E].

    Pinned by: exact math.fsum of sampled entries; W_g = identity reproduces x.
    """
    X = widen(x, dtype)
    W = widen(w_g, dtype)
    _finite(X, W, bias)
    L = X @ W
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return L


def softmax_row(l: np.ndarray) -> np.ndarray:
    """Softmax over one token's logits, [Router] step 2, in float64."""
    l = np.asarray(l, dtype=np.float64)
    z = np.exp(l - l.max())
    return z / z.sum()


# ----------------------------------------------------------------- ranking

def token_order(l32: np.ndarray) -> np.ndarray:
    """All experts of one token, best first (reading R1).

    Primary key: logit descending; secondary: expert index ascending.
    Negating a float32 is exact and maps -0.0/+0.0 to values that compare
    equal, so the index decides between them.

    Pinned by: brute-force comparison of every selected/unselected pair, and
    the hand-worked routing examples.
    """
    l32 = np.asarray(l32, dtype=np.float32)
    idx = np.arange(l32.shape[0])
    # lexsort sorts by the last key first.
    return np.lexsort((idx, -l32.astype(np.float64)))


def _first_in(order: np.ndarray, allowed: np.ndarray, count: int) -> list:
    out = []
    for e in order:
        if allowed[e]:
            out.append(int(e))
            if len(out) == count:
                break
    return out


def _ids_matrix(sel_lists, k: int) -> np.ndarray:
    ids = np.full((len(sel_lists), k), -1, dtype=np.int32)
    for t, s in enumerate(sel_lists):
        ids[t, :len(s)] = s
    return ids


# --------------------------------------------------------------- policies

def select_topk(L32: np.ndarray, k: int) -> np.ndarray:
    """Standard per-token top-k ([Router] step 3). ids [B, k].

    Pinned by: brute force over k-subsets; equals oea(k0 = k) and budget(E).
    """
    return _ids_matrix([list(token_order(l)[:k]) for l in L32], k)


def oea_active_set(L32: np.ndarray, k0: int) -> np.ndarray:
    """[OEA]: the union over the batch of each token's k0 most important
    experts (reading R4). Boolean mask [E].

    Pinned by: brute force (smallest set holding every token's top-k0),
    |S(k0)| <= |S_topk|, S(k0) subset of S(k0+1).
    """
    B, E = L32.shape
    S = np.zeros(E, dtype=bool)
    for l in L32:
        S[token_order(l)[:k0]] = True
    return S


def select_oea(L32: np.ndarray, k: int, k0: int) -> np.ndarray:
    """[OEA] piggyback re-route (reading R4): keep the top-k0, then fill up to
    k slots with the token's highest-scored experts among those the batch
    already loads. ids [B, k], -1 padded.

    Pinned by: oea(k) == topk; each token keeps its own top-k0; every expert
    of S gets a token; brute force (retained mass is maximal within S).
    """
    if not 1 <= k0 <= k:
        raise ValueError("k0 must be in [1, k]")
    S = oea_active_set(L32, k0)
    return _ids_matrix([_first_in(token_order(l), S, k) for l in L32], k)


def budget_mass(L32: np.ndarray) -> np.ndarray:
    """[XShare] total gating score per expert: sum over tokens (in token
    order) of each token's full softmax (reading R5). float64 [E].

    Pinned by: sums to B; brute-force optimality of the top-m set.
    """
    M = np.zeros(L32.shape[1], dtype=np.float64)
    for l in L32:
        M += softmax_row(np.asarray(l, dtype=np.float32).astype(np.float64))
    return M


def budget_set(mass: np.ndarray, m: int) -> np.ndarray:
    """The m experts of largest mass, ties to the lower index, decided on the
    float32-rounded masses (reading R2). Boolean mask [E]."""
    m32 = np.asarray(mass, dtype=np.float64).astype(np.float32)
    order = np.lexsort((np.arange(m32.shape[0]), -m32.astype(np.float64)))
    S = np.zeros(m32.shape[0], dtype=bool)
    S[order[:m]] = True
    return S


def select_budget(L32: np.ndarray, k: int, m: int, mass=None) -> np.ndarray:
    """budget(m): [XShare] modular objective with a cardinality budget
    (reading R5). ids [B, k], -1 padded.

    Pinned by: brute force over all m-subsets (total gating score is
    maximal); budget(E) == topk; the (k/m) bound on retained top-k mass.
    """
    B, E = L32.shape
    if not 1 <= m <= E:
        raise ValueError("m must be in [1, E]")
    if mass is None:
        mass = budget_mass(L32)
    S = budget_set(mass, m)
    return _ids_matrix([_first_in(token_order(l), S, k) for l in L32], k)


def greedy_retained_set(L32: np.ndarray, k: int, m: int, prefer=None,
                        term_rel: float = 0.0) -> np.ndarray:
    """Greedy maximisation of the retained top-k gating mass
    F(S) = sum_t (sum of token t's k largest probabilities inside S), one
    expert at a time ([XShare] abstract: batch-aware selection solved
    greedily for the largest total gating score). Marginal gains are compared
    on float32-rounded values, ties to the lower index (reading R2).
    Boolean mask [E].

    Near ties. An implementation that computes the probabilities and gains
    in float32 can order two gains that differ only by rounding the other
    way, and both greedy runs are then correct (the reading taken for budget's
    mass near-ties). Given ``prefer`` (boolean [E], the set such an
    implementation chose) and ``term_rel`` (a bound on the relative error of
    each of its float32 probabilities), a round whose best candidate is not in
    ``prefer`` takes instead the lowest-index candidate in ``prefer`` whose
    gain is within the rounding bound of the best. The bound of candidate e is
    term_rel' * sum over tokens with p_t[e] >= thr_t / 2 of (p_t[e] + thr_t)
    (the error of each term max(0, p_t[e] - thr_t), term_rel' = term_rel +
    2^-24 for the subtraction; tokens further below their threshold add 0 on
    both sides) plus (B - 1) 2^-24 gain_e (a float32 sum of B terms), where
    thr_t is token t's k-th largest probability inside S (0 while S holds
    fewer than k). Two gains are near-tied when they differ by at most the
    sum of their bounds. Without ``prefer`` the run is the exact greedy.

    Pinned by: hand-worked examples (greedy differs from budget(m) and from
    the exhaustive optimum), brute force on tiny inputs (1 - 1/e bound), and
    equality with budget(m) when m <= k (F is then modular on |S| <= k).
    """
    B, E = L32.shape
    P = np.stack([softmax_row(np.asarray(l, np.float32).astype(np.float64)) for l in L32])
    S = np.zeros(E, dtype=bool)
    u = 2.0 ** -24

    def F(mask):
        tot = 0.0
        for t in range(B):
            v = np.sort(P[t][mask])[::-1][:k]
            tot += v.sum()
        return tot

    def thresholds(mask):
        thr = np.zeros(B)
        for t in range(B):
            v = np.sort(P[t][mask])[::-1]
            if v.shape[0] >= k:
                thr[t] = v[k - 1]
        return thr

    base = 0.0
    for _ in range(m):
        best_e, best_gain = -1, None
        gains = {}
        for e in range(E):
            if S[e]:
                continue
            S[e] = True
            gain = np.float32(F(S) - base)
            S[e] = False
            gains[e] = float(gain)
            if best_gain is None or gain > best_gain:
                best_e, best_gain = e, gain
        if prefer is not None and not prefer[best_e]:
            thr = thresholds(S)
            rel = term_rel + u

            def bound(e):
                near = P[:, e] >= thr / 2
                return rel * float(np.sum((P[:, e] + thr)[near])) + (B - 1) * u * gains[e]

            tb = bound(best_e)
            for e in sorted(gains):
                if prefer[e] and gains[best_e] - gains[e] <= tb + bound(e):
                    best_e = e
                    break
        S[best_e] = True
        base = F(S)
    return S


def select_greedy(L32: np.ndarray, k: int, m: int, prefer=None, term_rel: float = 0.0) -> np.ndarray:
    """greedy(m): each token takes the first min(k, m) experts of its own
    order inside the greedy set. ids [B, k], -1 padded. ``prefer`` and
    ``term_rel`` as in greedy_retained_set."""
    S = greedy_retained_set(L32, k, m, prefer, term_rel)
    return _ids_matrix([_first_in(token_order(l), S, k) for l in L32], k)


def request_sets(L32: np.ndarray, m: int, m_r: int, g: int, mass=None) -> np.ndarray:
    """hier(m, m_r, g), the request level (reading R8): boolean [R, E], row r
    the m_r experts of the batch's budget(m) set with the largest mass summed
    over request r's tokens r*g .. r*g+g-1 (the last request may be shorter),
    decided on float32-rounded sums, ties to the lower index.

    Pinned by: brute force over every m_r-subset of S_b (each row maximises
    the request's total gating score); m_r = m gives S_b for every request;
    one request (g >= B) gives budget(m_r); rows lie inside S_b.
    """
    B, E = L32.shape
    if not 1 <= m <= E or not 1 <= m_r <= m or g < 1:
        raise ValueError("need 1 <= m_r <= m <= E and g >= 1")
    if mass is None:
        mass = budget_mass(L32)
    Sb = budget_set(mass, m)
    R = -(-B // g)
    out = np.zeros((R, E), dtype=bool)
    for r in range(R):
        Mr = np.zeros(E, dtype=np.float64)
        for t in range(r * g, min(B, r * g + g)):
            Mr += softmax_row(np.asarray(L32[t], dtype=np.float32).astype(np.float64))
        m32 = Mr.astype(np.float32).astype(np.float64)
        cand = [e for e in range(E) if Sb[e]]
        cand.sort(key=lambda e: (-m32[e], e))
        out[r, cand[:m_r]] = True
    return out


def select_hier(L32: np.ndarray, k: int, m: int, m_r: int, g: int, mass=None) -> np.ndarray:
    """hier(m, m_r, g) (reading R8): each token takes the first min(k, m_r)
    experts of its own order inside its request's set. ids [B, k], -1 padded.

    Pinned by: g = 1 with m_r >= k equals budget(m); g >= B equals
    budget(m_r); m_r = m equals budget(m) for any g; each token's selection
    is the top of its own order inside its request's set.
    """
    S = request_sets(L32, m, m_r, g, mass)
    return _ids_matrix([_first_in(token_order(l), S[t // g], k) for t, l in enumerate(L32)], k)


def lynx_bin_width(E: int, k: int) -> np.float32:
    """AffinityBinning width (reading R9): ln(E / k) rounded to float32."""
    return np.float32(math.log(E / k))


def lynx_scores(L32: np.ndarray, k: int) -> np.ndarray:
    """Adaptive expert scores (reading R9): for every token and each of its
    k best experts, 2^(k - 1 - bin) with bin the token's confidence bin for
    that expert. int64 [E].

    Pinned by: a hand-worked example; invariance under token permutation.
    """
    B, E = L32.shape
    w = lynx_bin_width(E, k)
    thr = [np.float32(np.float32(i) * w) for i in range(1, k)]
    score = np.zeros(E, dtype=np.int64)
    for l in np.asarray(L32, dtype=np.float32):
        o = token_order(l)
        top = np.float32(l[o[0]])
        for j in range(k):
            delta = np.float32(top - np.float32(l[o[j]]))
            b = sum(1 for t in thr if delta >= t)
            score[o[j]] += 1 << (k - 1 - b)
    return score


def lynx_critical_set(L32: np.ndarray, k: int, m: int) -> np.ndarray:
    """The critical set C of lynx(m) (reading R9). Boolean mask [E].

    Pinned by: C holds every rank-0 expert; |C| = min(max(m, |R0|), |U|)
    with U the union of the tokens' top-k; C(m) is inside C(m + 1);
    m <= |R0| gives R0.
    """
    B, E = L32.shape
    score = lynx_scores(L32, k)
    C = np.zeros(E, dtype=bool)
    named = np.zeros(E, dtype=bool)
    for l in np.asarray(L32, dtype=np.float32):
        o = token_order(l)
        C[o[0]] = True
        named[o[:k]] = True
    n0 = int(C.sum())
    rest = [e for e in range(E) if named[e] and not C[e]]
    rest.sort(key=lambda e: (-score[e], e))
    C[rest[:max(0, m - n0)]] = True
    return C


def select_lynx(L32: np.ndarray, k: int, m: int) -> np.ndarray:
    """lynx(m) (reading R9): each token takes the first k experts of its own
    order inside the critical set. ids [B, k].

    Pinned by: exactly k distinct experts per token with rank 0 in slot 0;
    m >= |U| equals topk; k <= m <= |R0| equals oea(k0 = 1).
    """
    B, E = L32.shape
    if not 1 <= k <= m <= E:
        raise ValueError("lynx needs 1 <= k <= m <= E")
    C = lynx_critical_set(L32, k, m)
    return _ids_matrix([_first_in(token_order(l), C, k) for l in L32], k)


def select(L32: np.ndarray, policy: str, k: int, k0: int = 0, m: int = 0, g: int = 0):
    """Dispatch on policy name. Returns (ids [B,k] int32, mass or None).
    hier takes m (batch budget), k0 (the request budget m_r) and g (tokens per
    request)."""
    L32 = np.asarray(L32, dtype=np.float32)
    _finite(L32)
    B, E = L32.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    if policy == POLICY_TOPK:
        return select_topk(L32, k), None
    if policy == POLICY_OEA:
        return select_oea(L32, k, k0), None
    if policy == POLICY_BUDGET:
        M = budget_mass(L32)
        return select_budget(L32, k, m, M), M
    if policy == POLICY_GREEDY:
        return select_greedy(L32, k, m), None
    if policy == POLICY_HIER:
        M = budget_mass(L32)
        return select_hier(L32, k, m, k0, g, M), M
    if policy == POLICY_LYNX:
        return select_lynx(L32, k, m), None
    raise ValueError(policy)


# ------------------------------------------------------------ gate weights

def gate_weights(L32: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Renormalised gate weights (reading R3): softmax over the selected
    logits only, float64 [B, k], 0 on empty slots.

    Pinned by: sums to 1; equals p[sel] / p[sel].sum() from the full softmax.
    """
    B, k = ids.shape
    W = np.zeros((B, k), dtype=np.float64)
    for t in range(B):
        sel = [int(e) for e in ids[t] if e >= 0]
        if not sel:
            continue
        v = np.asarray(L32[t], dtype=np.float32).astype(np.float64)[sel]
        z = np.exp(v - v[0])  # slot 0 holds the largest selected logit
        W[t, :len(sel)] = z / z.sum()
    return W


# -------------------------------------------------------------- compaction

def compact(ids: np.ndarray, E: int) -> dict:
    """Active expert list and per-expert token lists ([Lynx] section 2.2: the
    batch activates a consolidated set; only it is streamed).

    active[E]     ascending expert ids with >= 1 token, then -1
    n_active      number of such experts
    offsets[E+1]  CSR offsets over the active list, padded with the total
    pair_token/pair_slot [B*k]  tokens ascending within each expert, then -1

    Pinned by: pairs are a permutation of the non-empty slots; the active
    list is the sorted union.
    """
    B, k = ids.shape
    used = np.zeros(E, dtype=bool)
    for t in range(B):
        for j in range(k):
            if ids[t, j] >= 0:
                used[ids[t, j]] = True
    active = [e for e in range(E) if used[e]]
    offsets = [0]
    ptok, pslot = [], []
    for e in active:
        for t in range(B):
            for j in range(k):
                if ids[t, j] == e:
                    ptok.append(t)
                    pslot.append(j)
        offsets.append(len(ptok))
    n = len(active)
    out_active = np.full(E, -1, dtype=np.int32)
    out_active[:n] = active
    out_off = np.full(E + 1, offsets[-1], dtype=np.int32)
    out_off[:n + 1] = offsets
    out_tok = np.full(B * k, -1, dtype=np.int32)
    out_slot = np.full(B * k, -1, dtype=np.int32)
    out_tok[:len(ptok)] = ptok
    out_slot[:len(pslot)] = pslot
    return {"n_active": n, "active": out_active, "offsets": out_off,
            "pair_token": out_tok, "pair_slot": out_slot}


# --------------------------------------------------------------------- FFN

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z) (reading R6)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x, ids, W, w_gate, w_up, w_down, dtype: str, tokens=None) -> np.ndarray:
    """Weighted sum of SwiGLU experts per token (reading R6), streaming only
    the experts some token selected. float64 [B, d]; rows not in ``tokens``
    (when given) are left zero.

    Pinned by: one expert reduces to a dense SwiGLU from plain matmuls;
    outputs are linear in D; experts no token selected do not matter; and
    each slot's weight multiplies its own expert's output (distinct experts
    whose down matrices are distinct scales of one matrix, hand-worked and
    over every policy), which a permutation of a token's weights fails.
    """
    X = widen(x, dtype)
    B, d = X.shape
    Y = np.zeros((B, d), dtype=np.float64)
    want = np.ones(B, dtype=bool) if tokens is None else np.isin(np.arange(B), tokens)
    needed = sorted({int(e) for t in range(B) if want[t] for e in ids[t] if e >= 0})
    for e in needed:
        G = widen(w_gate[e], dtype)
        U = widen(w_up[e], dtype)
        D = widen(w_down[e], dtype)
        for t in range(B):
            if not want[t]:
                continue
            for j in range(ids.shape[1]):
                if ids[t, j] == e:
                    h = silu(X[t] @ G) * (X[t] @ U)
                    Y[t] += W[t, j] * (h @ D)
    return Y


# ------------------------------------------------------------------- layer

def moe_layer(x, w_g, bias, w_gate, w_up, w_down, dtype: str, policy: str,
              k: int, k0: int = 0, m: int = 0, tokens=None, g: int = 0) -> dict:
    """The whole decode MoE layer: router, selection, weights, compaction,
    expert FFN. Selection runs on the float32-rounded logits (reading R2)."""
    L = router_logits(x, w_g, bias, dtype)
    L32 = L.astype(np.float32)
    ids, mass = select(L32, policy, k, k0, m, g)
    W = gate_weights(L32, ids)
    c = compact(ids, L.shape[1])
    y = expert_ffn(x, ids, W, w_gate, w_up, w_down, dtype, tokens)
    out = {"logits": L, "logits32": L32, "ids": ids, "w": W, "mass": mass, "y": y}
    out.update(c)
    return out
