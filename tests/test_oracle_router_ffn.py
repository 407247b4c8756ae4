"""Pins of the oracle's router product and SwiGLU expert FFN.

The router and FFN have no printed worked example on the pages, so they are
pinned by exact summation (math.fsum), special cases that reduce to textbook
formulas or plain matmuls, closed forms of SiLU, and structural invariants
(linearity in D, independence from unselected experts).
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as orc
from aware_expert_routing_amd.workloads import (CONFIGS, bf16_bits_from_f32, f32_from_bf16_bits,
                                                make_hidden, make_layer, make_router)


def _bf16(a):
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


# --------------------------------------------------------------- router

@pytest.mark.parametrize("cfg", ["tiny_f32", "lynx_bf16"])
def test_router_matches_exact_fsum(cfg):
    c = CONFIGS[cfg]
    rng = np.random.default_rng(0)
    x = make_hidden(c, 4, seed=1)
    w, b = make_router(c, seed=1)
    L = orc.router_logits(x, w, b, c.dtype)
    xf = f32_from_bf16_bits(x) if c.dtype == "bf16" else x
    wf = f32_from_bf16_bits(w) if c.dtype == "bf16" else w
    for _ in range(40):
        t, e = rng.integers(0, 4), rng.integers(0, c.E)
        # products of two float32 values are exact in float64; fsum is exact
        exact = math.fsum([float(xf[t, i]) * float(wf[i, e]) for i in range(c.d)] + [float(b[e])])
        assert abs(L[t, e] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_router_identity_reproduces_hidden():
    d = 64
    x = np.random.default_rng(1).standard_normal((5, d)).astype(np.float32)
    L = orc.router_logits(x, np.eye(d, dtype=np.float32), None, "f32")
    assert np.array_equal(L, x.astype(np.float64))
    xb = _bf16(x)
    Lb = orc.router_logits(xb, _bf16(np.eye(d)), None, "bf16")
    assert np.array_equal(Lb, f32_from_bf16_bits(xb).astype(np.float64))


def test_router_bias_is_added_per_expert():
    d, E = 32, 8
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, d)).astype(np.float32)
    w = np.zeros((d, E), dtype=np.float32)
    b = np.arange(E, dtype=np.float32) - 3.5
    L = orc.router_logits(x, w, b, "f32")
    assert np.array_equal(L, np.broadcast_to(b.astype(np.float64), (3, E)))


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    v = orc.widen(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0
    assert math.copysign(1.0, v[3]) == -1.0
    assert v[4] == 3.140625
    assert v[5] == float.fromhex("0x1.fep+127")
    with pytest.raises(TypeError):
        orc.widen(np.zeros(2, np.float32), "bf16")


# ----------------------------------------------------------------- SiLU

def test_silu_closed_forms():
    z = np.array([-30.0, -2.5, -1.0, 0.0, 0.5, 1.0, 4.0, 40.0])
    s = orc.silu(z)
    assert s[3] == 0.0
    # SiLU(z) = z * (1 + tanh(z/2)) / 2, the logistic function written with tanh
    np.testing.assert_allclose(s, z * (1 + np.tanh(z / 2)) / 2, rtol=1e-13, atol=1e-15)
    # SiLU(-z) = SiLU(z) - z
    np.testing.assert_allclose(orc.silu(-z), s - z, rtol=1e-12, atol=1e-12)
    assert abs(s[-1] - 40.0) < 1e-15 and abs(s[0]) < 3e-12
    assert orc.silu(np.array([-1000.0]))[0] == 0.0  # no overflow error, limit 0


# ------------------------------------------------------------------ FFN

def _tiny(E=4, d=48, I=24, B=5, dtype="f32", seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, d)).astype(np.float32)
    G = (0.2 * rng.standard_normal((E, d, I))).astype(np.float32)
    U = (0.2 * rng.standard_normal((E, d, I))).astype(np.float32)
    D = (0.2 * rng.standard_normal((E, I, d))).astype(np.float32)
    wg = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        return _bf16(x), _bf16(wg), _bf16(G), _bf16(U), _bf16(D)
    return x, wg, G, U, D


def _dense_swiglu(x64, G64, U64, D64):
    g = x64 @ G64
    return (g / (1 + np.exp(-g)) * (x64 @ U64)) @ D64


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_dense_swiglu(dtype):
    x, wg, G, U, D = _tiny(E=1, dtype=dtype)
    out = orc.moe_layer(x, wg, None, G, U, D, dtype, "topk", k=1)
    assert np.all(out["ids"] == 0) and np.all(out["w"] == 1.0)
    ref = _dense_swiglu(orc.widen(x, dtype), orc.widen(G[0], dtype), orc.widen(U[0], dtype),
                        orc.widen(D[0], dtype))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("policy,kw", [("topk", {}), ("oea", {"k0": 1}), ("budget", {"m": 2}),
                                       ("greedy", {"m": 3})])
def test_identical_experts_are_dense_swiglu(policy, kw):
    """All experts equal: any selection mixes one function with weights that sum
    to 1, so the layer equals one dense SwiGLU FFN."""
    x, wg, G, U, D = _tiny(E=6)
    G[:] = G[0]
    U[:] = U[0]
    D[:] = D[0]
    out = orc.moe_layer(x, wg, None, G, U, D, "f32", policy, k=3, **kw)
    ref = _dense_swiglu(x.astype(np.float64), G[0].astype(np.float64), U[0].astype(np.float64),
                        D[0].astype(np.float64))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)


def test_gate_and_up_roles():
    """SiLU applies to x G, not x U: with U's output held at 1, y = SiLU(xG) D."""
    d, I = 2, 1
    x = np.array([[1.0, 2.0]], dtype=np.float32)
    G = np.array([[[1.0], [0.5]]], dtype=np.float32)      # x G = 2
    U = np.array([[[0.5], [0.25]]], dtype=np.float32)     # x U = 1
    D = np.array([[[1.0, -2.0]]], dtype=np.float32)
    wg = np.zeros((d, 1), dtype=np.float32)
    out = orc.moe_layer(x, wg, None, G, U, D, "f32", "topk", k=1)
    s2 = 2 * (1 + math.tanh(1.0)) / 2  # SiLU(2)
    np.testing.assert_allclose(out["y"][0], [s2, -2 * s2], rtol=1e-14)
    # swapping the roles changes the result: SiLU(1) * 2 != SiLU(2) * 1
    out2 = orc.moe_layer(x, wg, None, U, G, D, "f32", "topk", k=1)
    assert abs(out2["y"][0, 0] - s2) > 0.1


def test_ffn_linear_in_down_projection():
    x, wg, G, U, D = _tiny(E=5)
    a = orc.moe_layer(x, wg, None, G, U, D, "f32", "oea", k=2, k0=1)["y"]
    b = orc.moe_layer(x, wg, None, G, U, (2 * D).astype(np.float32), "f32", "oea", k=2, k0=1)["y"]
    assert np.array_equal(b, 2 * a)  # power-of-two scaling is exact
    z = orc.moe_layer(x, wg, None, G, U, np.zeros_like(D), "f32", "oea", k=2, k0=1)["y"]
    assert np.all(z == 0)


@pytest.mark.parametrize("policy,kw", [("topk", {}), ("oea", {"k0": 1}), ("budget", {"m": 3})])
def test_unselected_experts_do_not_matter(policy, kw):
    """Only the active experts are read: overwriting every other expert's
    weights leaves the outputs bit-identical."""
    x, wg, G, U, D = _tiny(E=8, B=3)
    a = orc.moe_layer(x, wg, None, G, U, D, "f32", policy, k=2, **kw)
    inactive = [e for e in range(8) if e not in a["active"][:a["n_active"]]]
    assert inactive
    G2, U2, D2 = G.copy(), U.copy(), D.copy()
    G2[inactive] = 1e3
    U2[inactive] = -7
    D2[inactive] = 5
    b = orc.moe_layer(x, wg, None, G2, U2, D2, "f32", policy, k=2, **kw)
    assert np.array_equal(a["y"], b["y"])


def test_topk_tokens_are_independent():
    """Under plain top-k a token's output depends on that token alone."""
    x, wg, G, U, D = _tiny(E=8, B=6)
    full = orc.moe_layer(x, wg, None, G, U, D, "f32", "topk", k=3)["y"]
    for t in range(6):
        one = orc.moe_layer(x[t:t + 1], wg, None, G, U, D, "f32", "topk", k=3)["y"]
        np.testing.assert_array_equal(one[0], full[t])


def test_sampled_tokens_match_full_layer():
    x, wg, G, U, D = _tiny(E=8, B=6)
    full = orc.moe_layer(x, wg, None, G, U, D, "f32", "oea", k=3, k0=1)
    part = orc.moe_layer(x, wg, None, G, U, D, "f32", "oea", k=3, k0=1, tokens=[1, 4])
    np.testing.assert_array_equal(part["y"][[1, 4]], full["y"][[1, 4]])
    assert np.all(part["y"][[0, 2, 3, 5]] == 0)


def test_tiny_config_layer_runs_and_is_finite():
    c = CONFIGS["tiny_f32"]
    inp = make_layer(c, 4)
    for pol, kw in (("topk", {}), ("oea", {"k0": 2}), ("budget", {"m": 4}), ("budget", {"m": 8})):
        out = orc.moe_layer(inp["x"], inp["w_g"], inp["bias"], inp["w_gate"], inp["w_up"],
                            inp["w_down"], c.dtype, pol, c.k, **kw)
        assert np.all(np.isfinite(out["y"]))
        assert 1 <= out["n_active"] <= min(c.E, 4 * c.k)


def test_oea_reduces_active_experts_on_skewed_workload():
    """On the Qwen3-30B-shaped workload at batch 16, oea with small k0 loads
    fewer experts than top-k (the effect the OEA abstract reports)."""
    c = CONFIGS["qwen3_30b_bf16"]
    x = make_hidden(c, 16)
    w, b = make_router(c)
    L32 = orc.router_logits(x, w, b, c.dtype).astype(np.float32)
    n = {k0: orc.compact(orc.select(L32, "oea", 8, k0=k0)[0], c.E)["n_active"] for k0 in range(1, 9)}
    n_topk = orc.compact(orc.select(L32, "topk", 8)[0], c.E)["n_active"]
    assert n[8] == n_topk
    assert all(n[a] <= n[a + 1] for a in range(1, 8))
    assert n[2] < n_topk


def test_slot_weights_pair_with_their_experts_hand_worked():
    """Two experts with the same gate/up and different down projections, one
    token, k = 2. x = (1, 0), W_g puts logit ln 3 on expert 0 and 0 on expert
    1, so the renormalised weights are 3/4 and 1/4. Both experts have
    x G = 2 and x U = 1, so h = SiLU(2); D_0 = [1, 0] and D_1 = [0, 1] route
    h to different output columns. y = SiLU(2) * (3/4, 1/4): each weight must
    multiply its own expert's output."""
    x = np.array([[1.0, 0.0]], dtype=np.float32)
    wg = np.array([[math.log(3.0), 0.0], [0.0, 0.0]], dtype=np.float32)
    G = np.array([[[2.0], [0.0]]] * 2, dtype=np.float32)
    U = np.array([[[1.0], [0.0]]] * 2, dtype=np.float32)
    D = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], dtype=np.float32)
    out = orc.moe_layer(x, wg, None, G, U, D, "f32", "topk", k=2)
    assert out["ids"].tolist() == [[0, 1]]
    s2 = 2 * (1 + math.tanh(1.0)) / 2  # SiLU(2) = 2 / (1 + e^-2)
    # ln 3 rounded to float32 moves the weights by about 1e-8
    np.testing.assert_allclose(out["y"][0], [0.75 * s2, 0.25 * s2], rtol=1e-7)


@pytest.mark.parametrize("policy,kw", [("topk", {}), ("oea", {"k0": 1}), ("budget", {"m": 4}),
                                       ("greedy", {"m": 3})])
def test_slot_weights_pair_with_their_experts(policy, kw):
    """Experts that share G and U and whose down projections are D scaled by
    2^e: expert e computes 2^e f(x) with f one dense SwiGLU. So
    y[t] = (sum_j w[t,j] 2^{e_j}) f(x_t), where w is the softmax of the
    selected logits computed here with scipy. Distinct logits give distinct
    weights and distinct scales, so a weight paired with another slot's
    expert changes the factor."""
    from scipy.special import softmax as sp_softmax
    E, B, k = 6, 5, 3
    x, wg, G, U, D = _tiny(E=E, B=B)
    G[:] = G[0]
    U[:] = U[0]
    D = np.stack([D[0] * np.float32(2.0 ** e) for e in range(E)]).astype(np.float32)
    out = orc.moe_layer(x, wg, None, G, U, D, "f32", policy, k=k, **kw)
    f = _dense_swiglu(x.astype(np.float64), G[0].astype(np.float64), U[0].astype(np.float64),
                      D[0].astype(np.float64))
    L32 = out["logits32"]
    for t in range(B):
        sel = [int(e) for e in out["ids"][t] if e >= 0]
        assert len(sel) >= 2, "the pin needs tokens with several experts"
        p = sp_softmax(L32[t].astype(np.float64))[sel]
        w = p / p.sum()
        assert len(set(np.round(w, 12))) == len(w), "weights must be distinct"
        c = float(np.dot(w, [2.0 ** e for e in sel]))
        np.testing.assert_allclose(out["y"][t], c * f[t], rtol=1e-11, atol=1e-13)
