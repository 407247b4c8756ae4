"""Seeded input generator: determinism, rounding, prefix/subset properties and
the distributions the workloads describe."""
import hashlib

import numpy as np
import pytest
import torch

from aware_expert_routing_amd.workloads import (CONFIGS, bf16_bits_from_f32, f32_from_bf16_bits,
                                                make_expert_weights, make_hidden, make_layer,
                                                make_logits, make_router)


def test_bf16_rounding_matches_torch():
    """torch's float32 -> bfloat16 conversion rounds to nearest-even."""
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40], np.float32)])
    # exact ties: low 16 bits 0x8000, with even and odd kept parts
    ties = (np.arange(1000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)) + np.uint32(0x3F000000)
    a = np.concatenate([a, ties.view(np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(a), ref)
    back = f32_from_bf16_bits(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_deterministic():
    c = CONFIGS["tiny_f32"]
    a = make_layer(c, 4, seed=0)
    b = make_layer(c, 4, seed=0)
    for k in a:
        if a[k] is None:
            continue
        assert np.array_equal(a[k], b[k])
    other = make_layer(c, 4, seed=1)
    assert not np.array_equal(a["x"], other["x"])


def test_generator_frozen_hash():
    """The tiny workload's bytes are frozen; a change to the generator shows here."""
    c = CONFIGS["tiny_f32"]
    a = make_layer(c, 4, seed=0)
    h = hashlib.sha256()
    for k in ("x", "w_g", "bias", "w_gate", "w_up", "w_down"):
        h.update(np.ascontiguousarray(a[k]).tobytes())
    assert h.hexdigest() == FROZEN_TINY_SHA256


FROZEN_TINY_SHA256 = "18f1cdb6c5450836895cd873aa244139bfec9cc744a6b2c02551a9fba7d870c7"


def test_hidden_prefix_property():
    c = CONFIGS["qwen3_30b_bf16"]
    x16 = make_hidden(c, 16)
    x32 = make_hidden(c, 32)
    assert np.array_equal(x32[:16], x16)


def test_expert_subset_is_bit_identical():
    c = CONFIGS["tiny_f32"]
    G, U, D = make_expert_weights(c)
    g, u, dn = make_expert_weights(c, experts=[7, 2])
    assert np.array_equal(g, G[[7, 2]]) and np.array_equal(u, U[[7, 2]]) and np.array_equal(dn, D[[7, 2]])


def test_distributions():
    c = CONFIGS["lynx_bf16"]
    w, b = make_router(c)
    wf = f32_from_bf16_bits(w)
    assert abs(wf.std() * np.sqrt(c.d) - 1.0) < 0.02
    assert abs(b.astype(np.float64).mean()) < 1e-5
    # rank-1 expert gets s * (mean ln r - ln 1)
    r = np.arange(1, c.E + 1, dtype=np.float64)
    assert np.isclose(b.max(), c.zipf_s * np.log(r).mean(), rtol=1e-6)
    assert np.isclose(b.min(), c.zipf_s * (np.log(r).mean() - np.log(c.E)), rtol=1e-6)
    G, U, D = make_expert_weights(c, experts=[0, 1])
    assert abs(f32_from_bf16_bits(G).std() - 0.02) < 2e-4
    x = f32_from_bf16_bits(make_hidden(c, 16))
    assert abs(x.std() - 1.0) < 0.02


def test_request_structure():
    c = CONFIGS["specdec_bf16"]
    x = f32_from_bf16_bits(make_hidden(c, 64)).astype(np.float64)
    xn = x / np.linalg.norm(x, axis=1, keepdims=True)
    same = [xn[4 * r] @ xn[4 * r + 1] for r in range(16)]
    diff = [xn[4 * r] @ xn[4 * r + 4] for r in range(15)]
    assert abs(np.mean(same) - 0.8) < 0.05
    assert abs(np.mean(diff)) < 0.1


def test_make_logits_kinds():
    L = make_logits(4, 16, kind="ties")
    assert np.any(np.signbit(L) & (L == 0)) and np.any(~np.signbit(L) & (L == 0))
    assert np.all(make_logits(3, 5, kind="flat") == 0)
