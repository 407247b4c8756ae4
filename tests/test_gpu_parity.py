"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Cases cover the five workload shapes at their configured batches and
policies, standalone selection on seeded logits (including exact ties and
signed zeros), ragged sizes, experts with more than 64 tokens, the maximum
envelope and degenerate layers. Expected values always come from the
oracle run on the same seeded inputs; tolerances are in gpu_helpers.
"""
import functools

import numpy as np
import pytest
import torch

from aware_expert_routing_amd import _lib as L
from aware_expert_routing_amd.workloads import (CONFIGS, LayerConfig, bf16_bits_from_f32,
                                                make_hidden, make_layer, make_logits)
from gpu_helpers import (Guarded, assert_batch_mass_close, assert_logits_close, assert_routing_equal,
                         assert_y_close, policy_args, routing_numpy, softmax_term_rel, to_dev,
                         weight_rtol_from_logits, y_to_f64)
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------- fixtures

@functools.lru_cache(maxsize=1)
def _layer_inputs(cname: str):
    """Full-size seeded weights for one config, on host and device (one config
    cached at a time to bound host memory)."""
    cfg = CONFIGS[cname]
    Bmax = max(cfg.batches)
    inp = make_layer(cfg, Bmax)
    dev = {k: to_dev(v, cfg.dtype) for k, v in inp.items()}
    return inp, dev


def _dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def _run_layer(cfg: LayerConfig, inp, dev, B: int, policy: str, k0: int, m: int, guard=True, g: int = 0):
    tdt = _dtype(cfg)
    x = dev["x"][:B].contiguous()
    pol = L.make_policy(policy, cfg.k, k0, m, g)
    r = L.Routing(B, cfg.E, cfg.k)
    ws = L.alloc_workspace(B, cfg.d, cfg.E, cfg.I, cfg.k, tdt)
    lg = Guarded((B, cfg.E), torch.float32, -7.0)
    y = Guarded((B, cfg.d), tdt, 3.0)
    L.moe_layer_decode(x, dev["w_g"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"], pol,
                       lg.t, r, y.t, ws)
    torch.cuda.synchronize()
    if guard:
        assert lg.intact() and y.intact(), "write past the end of an output buffer"
    _assert_sync_words_clear(ws)
    return lg.t.cpu().numpy(), routing_numpy(r), y.t


# Fixed counter region at the start of every workspace (byte offsets): barrier
# count (0), release word (128), error word (256), router + selection counter
# (384), router tile counters (512..1535), per-(strip, 16-token group)
# counters (from 2048: 128 strips x 16 groups, 128 bytes each), per gate/up
# tile slice counters (then 4096 of them, 64 bytes each).
_GRP_CNT = (2048, 2048 + 128 * 16 * 128)
_TILE_CNT = (_GRP_CNT[1], _GRP_CNT[1] + 4096 * 64)


def _assert_sync_words_clear(ws):
    """The FFN's grid-barrier count returns to zero, its error word stays
    zero (no bounded wait ran out), and every counter (router + selection,
    router tiles, per-group strips, gate/up tiles) is back at zero."""
    words = ws[:_TILE_CNT[1]].view(torch.int32).cpu().numpy()
    assert words[0] == 0, f"barrier count left at {words[0]}"
    assert words[64] == 0, "a bounded wait exceeded its limit"
    assert words[96] == 0, "the router + selection counter was left non-zero"
    assert not words[128:384].any(), "a router tile counter was left non-zero"
    assert not words[_GRP_CNT[0] // 4:_GRP_CNT[1] // 4].any(), "a per-group counter was left non-zero"
    assert not words[_TILE_CNT[0] // 4:_TILE_CNT[1] // 4].any(), "a gate/up tile counter was left non-zero"


def _oracle(cfg, inp, B, policy, k0, m, tokens=None, g=0):
    return orc.moe_layer(inp["x"][:B], inp["w_g"], inp["bias"], inp["w_gate"], inp["w_up"],
                         inp["w_down"], cfg.dtype, policy, cfg.k, k0, m, tokens=tokens, g=g)


def _greedy_ids(L32, k, m, g_ids, E):
    """The oracle's greedy on L32, taking near-tied gains the way the GPU did:
    where the GPU's set holds a candidate whose gain is within the float32
    rounding bound of the round's best, the oracle takes it."""
    prefer = np.zeros(E, dtype=bool)
    prefer[g_ids[g_ids >= 0]] = True
    return orc.select_greedy(L32, k, m, prefer=prefer,
                             term_rel=float(softmax_term_rel(L32).max()))


def _assert_routing_from_gpu_logits(Lg, rg, cfg, a):
    """The oracle's selection run on the GPU's own float32 logits reproduces
    the GPU routing bit for bit (budget ranks the GPU's batch masses, which
    must lie within the float32 error bound of the oracle's masses of the
    same logits; greedy accepts the GPU's choice only between gains that tie
    within their float32 error bound)."""
    if a["policy"] in ("budget", "hier"):
        M = orc.budget_mass(Lg)
        assert_batch_mass_close(rg["mass"], M, Lg)
        if a["policy"] == "budget":
            ids = orc.select_budget(Lg, cfg.k, a["m"], mass=rg["mass"])
        else:
            ids = orc.select_hier(Lg, cfg.k, a["m"], a["k0"], a["g"], mass=rg["mass"])
    elif a["policy"] == "greedy":
        ids = _greedy_ids(Lg, cfg.k, a["m"], rg["ids"], cfg.E)
    else:
        ids, _ = orc.select(Lg, a["policy"], cfg.k, a["k0"], a["m"])
    o = {"ids": ids, "w": orc.gate_weights(Lg, ids)}
    o.update(orc.compact(ids, cfg.E))
    assert_routing_equal(rg, o, "oracle on GPU logits")


def _layer_cases():
    cases = []
    for cname, cfg in CONFIGS.items():
        pols = [("topk", 0)] + [("oea", k0) for k0 in cfg.oea_k0] + [("budget", m) for m in cfg.budget_m]
        for B in cfg.batches:
            for pol, p in pols:
                if cname == "qwen3_30b_bf16" and pol == "oea" and B != 16 and p not in (1, 4):
                    continue  # full k0 sweep at B=16 only
                cases.append(pytest.param(cname, B, pol, p, id=f"{cname}-B{B}-{pol}{p or ''}"))
    return cases


# ------------------------------------------------------------ whole layer

def _greedy_layer_cases():
    return [pytest.param(c, B, "greedy", m, id=f"{c}-B{B}-greedy{m}")
            for c, B, m in (("tiny_f32", 4, 4), ("tiny_f32", 4, 8), ("lynx_bf16", 16, 24),
                            ("qwen3_30b_bf16", 16, 24), ("qwen3_30b_bf16", 16, 32),
                            ("specdec_bf16", 64, 32))]


def _hier_layer_cases():
    # (m, m_r, g): the speculative batch's own request structure (g = 4
    # drafts per request), and other batches grouped for coverage.
    return [pytest.param(c, B, "hier", p, id=f"{c}-B{B}-hier{p[0]}-{p[1]}-{p[2]}")
            for c, B, p in (("specdec_bf16", 64, (48, 12, 4)), ("specdec_bf16", 64, (32, 8, 4)),
                            ("specdec_bf16", 64, (64, 16, 4)), ("qwen3_30b_bf16", 16, (32, 8, 2)),
                            ("qwen3_30b_bf16", 32, (48, 10, 4)), ("lynx_bf16", 16, (24, 10, 4)),
                            ("tiny_f32", 4, (8, 4, 2)))]


def _lynx_layer_cases():
    return [pytest.param(c, B, "lynx", m, id=f"{c}-B{B}-lynx{m}")
            for c, B, m in (("tiny_f32", 4, 4), ("tiny_f32", 4, 10), ("lynx_bf16", 16, 24),
                            ("qwen3_30b_bf16", 16, 16), ("qwen3_30b_bf16", 16, 24),
                            ("qwen3_30b_bf16", 32, 32), ("specdec_bf16", 64, 32))]


@pytest.mark.parametrize("cname,B,policy,p",
                         _layer_cases() + _greedy_layer_cases() + _hier_layer_cases() + _lynx_layer_cases())
def test_layer_matches_oracle(cname, B, policy, p):
    cfg = CONFIGS[cname]
    inp, dev = _layer_inputs(cname)
    a = policy_args(policy, p)
    print(f"\n[case] {cname} B={B} {policy}{p}", flush=True)
    Lg, rg, y = _run_layer(cfg, inp, dev, B, a["policy"], a["k0"], a["m"], g=a["g"])
    o = _oracle(cfg, inp, B, a["policy"], a["k0"], a["m"], g=a["g"])
    assert_logits_close(Lg, o["logits"], cname)
    assert_routing_equal(rg, o, cname, weight_rtol_from_logits(Lg, o["logits"]))
    _assert_routing_from_gpu_logits(Lg, rg, cfg, a)
    # Every output row and column against the oracle.
    assert_y_close(y_to_f64(y), o["y"], cfg.dtype, f"{cname} B={B} {policy}{p}")


def test_layer_is_deterministic():
    cfg = CONFIGS["qwen3_30b_bf16"]
    inp, dev = _layer_inputs("qwen3_30b_bf16")
    outs = [_run_layer(cfg, inp, dev, 16, "oea", 2, 0) for _ in range(3)]
    for Lg, rg, y in outs[1:]:
        assert np.array_equal(Lg, outs[0][0])
        assert np.array_equal(rg["ids"], outs[0][1]["ids"])
        assert np.array_equal(rg["w"], outs[0][1]["w"])
        assert torch.equal(y, outs[0][2])


def test_workspace_reused_across_calls():
    """One workspace serves many calls in a row (the barrier words carry over)."""
    cfg = CONFIGS["qwen3_30b_bf16"]
    inp, dev = _layer_inputs("qwen3_30b_bf16")
    B = 16
    x = dev["x"][:B].contiguous()
    ws = L.alloc_workspace(B, cfg.d, cfg.E, cfg.I, cfg.k, torch.bfloat16)
    outs = []
    for pol, p in (("oea", 4), ("topk", 0), ("budget", 32), ("oea", 4), ("oea", 1)):
        a = policy_args(pol, p)
        r = L.Routing(B, cfg.E, cfg.k)
        lg = torch.empty((B, cfg.E), dtype=torch.float32, device="cuda")
        y = torch.empty((B, cfg.d), dtype=torch.bfloat16, device="cuda")
        L.moe_layer_decode(x, dev["w_g"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"],
                           L.make_policy(a["policy"], cfg.k, a["k0"], a["m"]), lg, r, y, ws)
        torch.cuda.synchronize()
        _assert_sync_words_clear(ws)
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[3])
    # Fresh workspace, same call: same bits.
    _, _, y_fresh = _run_layer(cfg, inp, dev, B, "oea", 1, 0)
    assert torch.equal(outs[4], y_fresh)


def test_workspace_shared_across_sizes():
    """One workspace (sized for the largest call) serves calls of different
    batch sizes in a row: each output equals a fresh workspace's, bit for bit."""
    cfg = CONFIGS["qwen3_30b_bf16"]
    inp, dev = _layer_inputs("qwen3_30b_bf16")
    Bmax = max(cfg.batches)
    ws = L.alloc_workspace(Bmax, cfg.d, cfg.E, cfg.I, cfg.k, torch.bfloat16)
    for B, pol, p in ((Bmax, "topk", 0), (1, "oea", 2), (16, "oea", 4), (4, "topk", 0), (Bmax, "oea", 3)):
        a = policy_args(pol, p)
        x = dev["x"][:B].contiguous()
        r = L.Routing(B, cfg.E, cfg.k)
        lg = torch.empty((B, cfg.E), dtype=torch.float32, device="cuda")
        y = torch.empty((B, cfg.d), dtype=torch.bfloat16, device="cuda")
        L.moe_layer_decode(x, dev["w_g"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"],
                           L.make_policy(a["policy"], cfg.k, a["k0"], a["m"]), lg, r, y, ws)
        torch.cuda.synchronize()
        _assert_sync_words_clear(ws)
        _, _, y_fresh = _run_layer(cfg, inp, dev, B, pol, a["k0"], a["m"])
        assert torch.equal(y, y_fresh), f"B={B} {pol}{p}"


@pytest.mark.parametrize("cname,B,m", [("lynx_bf16", 16, 24), ("tiny_f32", 4, 8)])
def test_route_select_ffn_equal_layer(cname, B, m):
    """The three standalone entry points reproduce the fused layer bit for bit
    (bf16: router and selection in one launch; float32: the same kernels)."""
    cfg = CONFIGS[cname]
    inp, dev = _layer_inputs(cname)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Lg, rg, y = _run_layer(cfg, inp, dev, B, "budget", 0, m)
    x = dev["x"][:B].contiguous()
    ws = L.alloc_workspace(B, cfg.d, cfg.E, cfg.I, cfg.k, tdt)
    lg = torch.empty((B, cfg.E), dtype=torch.float32, device="cuda")
    L.moe_route(x, dev["w_g"], dev["bias"], lg, ws)
    r = L.Routing(B, cfg.E, cfg.k)
    L.moe_select(lg, L.make_policy("budget", cfg.k, 0, m), r)
    y2 = torch.empty((B, cfg.d), dtype=tdt, device="cuda")
    L.moe_expert_ffn(x, dev["w_gate"], dev["w_up"], dev["w_down"], r, y2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(lg.cpu().numpy(), Lg)
    r2 = routing_numpy(r)
    for key in ("ids", "w", "active", "offsets", "pair_token", "pair_slot", "mass"):
        assert np.array_equal(r2[key], rg[key]), key
    assert torch.equal(y2, y)


# ------------------------------------------------------------- selection

_SEL_SHAPES = [(1, 128, 8), (4, 16, 4), (3, 8, 8), (16, 64, 8), (16, 128, 8), (64, 128, 8),
               (37, 100, 6), (40, 256, 8), (256, 256, 16), (128, 64, 1)]


def _sel_policies(E, k, B):
    out = [("topk", 0)]
    out += [("oea", k0) for k0 in sorted({1, max(1, k // 2), k})]
    out += [("budget", m) for m in sorted({1, max(1, k - 1), max(1, E // 4), E})]
    if B * E <= 64 * 128:  # the oracle's greedy re-sorts per candidate: keep it small
        out += [("greedy", m) for m in sorted({1, max(1, k - 1), max(1, E // 4)}
                                              | ({E} if B * E <= 128 else set()))]
    elif B <= 64:  # probabilities too many for LDS: one round past the first k
        out += [("greedy", k + 1)]
    mb = max(1, E // 2)
    out += [("hier", p) for p in sorted({(mb, max(1, min(mb, k // 2)), 2), (mb, min(mb, k + 2), 4),
                                          (E, max(1, k - 1), 1), (mb, max(1, mb // 2), B)})]
    out += [("lynx", m) for m in sorted({k, max(k, E // 4), max(k, E // 2), E})]
    return out


def _sel_cases():
    cases = []
    for (B, E, k) in _SEL_SHAPES:
        for kind in ("normal", "ties", "flat"):
            for pol, p in _sel_policies(E, k, B):
                tag = "-".join(map(str, p)) if isinstance(p, tuple) else (p or "")
                cases.append(pytest.param(B, E, k, kind, pol, p, id=f"B{B}-E{E}-k{k}-{kind}-{pol}{tag}"))
    return cases


@pytest.mark.parametrize("B,E,k,kind,policy,p", _sel_cases())
def test_select_matches_oracle(B, E, k, kind, policy, p):
    """Both sides rank the same float32 logits, so routing is bit-exact."""
    Lh = make_logits(B, E, seed=11, kind=kind)
    a = policy_args(policy, p)
    r = L.Routing(B, E, k)
    lg = to_dev(Lh, "f32")
    L.moe_select(lg, L.make_policy(a["policy"], k, a["k0"], a["m"], a["g"]), r)
    torch.cuda.synchronize()
    g = routing_numpy(r)
    ids, M = orc.select(Lh, a["policy"], k, a["k0"], a["m"], a["g"])
    o = {"ids": ids, "w": orc.gate_weights(Lh, ids)}
    o.update(orc.compact(ids, E))
    if policy == "greedy":
        ids_g = _greedy_ids(Lh, k, a["m"], g["ids"], E)
        assert np.array_equal(g["ids"], ids_g), "greedy set with the GPU's near-tie choices"
    if M is not None:
        assert_batch_mass_close(g["mass"], M, Lh)
        # Ranked on the GPU's own masses, the oracle's batch step must agree
        # exactly (masses that differ only by rounding may order differently).
        if policy == "budget":
            ids_g = orc.select_budget(Lh, k, a["m"], mass=g["mass"])
        else:
            ids_g = orc.select_hier(Lh, k, a["m"], a["k0"], a["g"], mass=g["mass"])
        assert np.array_equal(g["ids"], ids_g), f"{policy} set ranked on the GPU masses"
    assert_routing_equal(g, o, f"B{B} E{E} k{k} {kind} {policy}{p}")


# ------------------------------------------------------------- edge cases

def _custom_layer(B, d, E, I, k, dtype="bf16", seed=0, bias=None, wg_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, d)).astype(np.float32)
    wg = (wg_scale * rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    # Scaled so that x G, x U and y are O(1) at any d and I, as in the
    # configured workloads (the absolute output tolerance assumes that).
    G = (rng.standard_normal((E, d, I)) / np.sqrt(d)).astype(np.float32)
    U = (rng.standard_normal((E, d, I)) / np.sqrt(d)).astype(np.float32)
    D = (rng.standard_normal((E, I, d)) / np.sqrt(I)).astype(np.float32)
    b = None if bias is None else np.asarray(bias, dtype=np.float32)
    if dtype == "bf16":
        x, wg, G, U, D = (bf16_bits_from_f32(a) for a in (x, wg, G, U, D))
    inp = {"x": x, "w_g": wg, "bias": b, "w_gate": G, "w_up": U, "w_down": D}
    cfg = LayerConfig(name="custom", d=d, E=E, k=k, I=I, dtype=dtype, zipf_s=0.0, batches=(B,),
                      hidden="iid")
    return cfg, inp, {kk: to_dev(v, dtype) for kk, v in inp.items()}


@pytest.mark.parametrize("B,d,E,I,k,policy,p,dtype", [
    (5, 200, 10, 72, 3, "topk", 0, "bf16"),      # ragged d and I (not multiples of 64)
    (5, 200, 10, 72, 3, "oea", 1, "bf16"),
    (7, 136, 12, 40, 4, "budget", 3, "bf16"),
    (7, 136, 12, 40, 4, "oea", 2, "f32"),
    (1, 64, 1, 64, 1, "topk", 0, "bf16"),        # one expert: a dense SwiGLU
    (3, 64, 4, 64, 4, "topk", 0, "bf16"),        # k = E
    (256, 64, 256, 64, 16, "topk", 0, "bf16"),   # largest B, E and k
    (256, 64, 256, 64, 16, "oea", 3, "bf16"),
    (256, 64, 256, 64, 16, "budget", 40, "bf16"),
    (256, 64, 256, 64, 16, "hier", (96, 20, 8), "bf16"),  # 32 requests of 8 tokens
    (7, 136, 12, 40, 4, "hier", (9, 3, 3), "bf16"),      # ragged last request
    (9, 4096, 8, 64, 2, "topk", 0, "bf16"),      # deep reduction, several d slices
    (6, 448, 8, 256, 2, "topk", 0, "bf16"),      # whole gate/up tiles but strip 3 split over d, ragged d
    (16, 1024, 16, 512, 4, "oea", 2, "bf16"),    # the same with strips 3 and 7 of every expert split
    (24, 1024, 16, 512, 4, "topk", 0, "bf16"),   # the same split in the 32-token instantiation
])
def test_edge_layers(B, d, E, I, k, policy, p, dtype):
    cfg, inp, dev = _custom_layer(B, d, E, I, k, dtype)
    a = policy_args(policy, p)
    Lg, rg, y = _run_layer(cfg, inp, dev, B, a["policy"], a["k0"], a["m"], g=a["g"])
    o = _oracle(cfg, inp, B, a["policy"], a["k0"], a["m"], g=a["g"])
    assert_logits_close(Lg, o["logits"])
    assert_routing_equal(rg, o, w_rtol=weight_rtol_from_logits(Lg, o["logits"]))
    assert_y_close(y_to_f64(y), o["y"], dtype)


def test_expert_with_more_than_64_tokens():
    """A dominant expert receives all 150 tokens: several 64-token passes."""
    E = 16
    bias = np.zeros(E, np.float32)
    bias[5] = 30.0
    cfg, inp, dev = _custom_layer(150, 256, E, 128, 2, "bf16", bias=bias)
    for policy, p in (("topk", 0), ("oea", 1), ("budget", 2)):
        a = policy_args(policy, p)
        Lg, rg, y = _run_layer(cfg, inp, dev, 150, a["policy"], a["k0"], a["m"])
        o = _oracle(cfg, inp, 150, a["policy"], a["k0"], a["m"])
        assert_routing_equal(rg, o, w_rtol=weight_rtol_from_logits(Lg, o["logits"]))
        counts = np.diff(rg["offsets"][:rg["n_active"] + 1])
        assert counts.max() == 150
        assert_y_close(y_to_f64(y), o["y"], "bf16")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 15, 16, 17, 33, 64])
def test_token_counts_around_path_switch(T):
    """Experts with T tokens for T around the dot/MFMA switch and tile edges."""
    E = 4
    bias = np.array([40.0, 0.0, 0.0, 0.0], np.float32)  # every token takes expert 0 first
    cfg, inp, dev = _custom_layer(T, 512, E, 192, 1, "bf16", bias=bias, seed=T)
    Lg, rg, y = _run_layer(cfg, inp, dev, T, "topk", 0, 0)
    o = _oracle(cfg, inp, T, "topk", 0, 0)
    assert rg["n_active"] == 1
    assert_routing_equal(rg, o, w_rtol=weight_rtol_from_logits(Lg, o["logits"]))
    assert_y_close(y_to_f64(y), o["y"], "bf16")


def test_flat_router_ties():
    """W_g = 0 and no bias: every logit is 0, ties go to the lowest indices."""
    cfg, inp, dev = _custom_layer(8, 128, 16, 64, 4, "bf16", wg_scale=0.0)
    for policy, p in (("topk", 0), ("oea", 1), ("budget", 6)):
        a = policy_args(policy, p)
        Lg, rg, y = _run_layer(cfg, inp, dev, 8, a["policy"], a["k0"], a["m"])
        o = _oracle(cfg, inp, 8, a["policy"], a["k0"], a["m"])
        assert np.all(Lg == 0)
        assert_routing_equal(rg, o, w_rtol=weight_rtol_from_logits(Lg, o["logits"]))
        assert_y_close(y_to_f64(y), o["y"], "bf16")


def test_unselected_experts_are_not_read():
    """Overwriting the weights of inactive experts with NaN leaves y unchanged."""
    cfg = CONFIGS["qwen3_30b_bf16"]
    inp, dev = _layer_inputs("qwen3_30b_bf16")
    Lg, rg, y = _run_layer(cfg, inp, dev, 16, "oea", 2, 0)
    act = set(rg["active"][:rg["n_active"]].tolist())
    inactive = [e for e in range(cfg.E) if e not in act]
    g2, u2, d2 = (dev[k].clone() for k in ("w_gate", "w_up", "w_down"))
    for t in (g2, u2, d2):
        t[inactive] = float("nan")
    dev2 = dict(dev, w_gate=g2, w_up=u2, w_down=d2)
    _, rg2, y2 = _run_layer(cfg, inp, dev2, 16, "oea", 2, 0)
    assert torch.equal(y2, y)
    del g2, u2, d2, dev2
    torch.cuda.empty_cache()


def test_read_stream_reads_every_word():
    """moe_read_stream (the read-ceiling utility) folds exactly the words of
    each workgroup's contiguous block: its 1024 outputs equal the XOR of the
    same blocks computed on the host."""
    n16 = 1024 * 37 + 5  # 16-byte units, ragged over 1024 blocks
    g = np.random.default_rng(7)
    host = g.integers(0, 2**32, size=n16 * 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    L.moe_read_stream(src, out)
    torch.cuda.synchronize()
    per = -(-n16 // 1024)
    words = host.reshape(n16, 4)
    want = np.zeros(1024, dtype=np.uint32)
    for b in range(1024):
        blk = words[b * per:min((b + 1) * per, n16)]
        if len(blk):
            want[b] = np.bitwise_xor.reduce(blk.reshape(-1))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
