"""Seeded synthetic inputs for the decode-time MoE layer.

This module only draws inputs. It holds none of the layer's arithmetic (no
router product, no softmax, no selection, no FFN), so both the HIP path and
the CPU oracle can consume what it produces without sharing method code.

Workload shapes follow the models the pages name: the 64-expert, top-8 layer
of the Lynx explainer (Problem Statement), and the Qwen3-30B / Qwen3-235B
layers at batch 16 of the Opportunistic Expert Activation abstract; the
speculative-decoding batch follows the XShare abstract. No dataset is used:
every tensor is drawn from a seeded generator.

Readings of the distribution notation (the pages give none; the workload
descriptions do):
  * ``W_g ~ N(0, 1/d)``: variance 1/d, so logits are O(1).
  * expert weights ``N(0, 0.02)``: standard deviation 0.02.
  * request means ``N(0, 0.5)``: standard deviation 0.5; token noise std 1.
  * speculative batch: request mean variance 0.8, per-token noise variance
    0.2, so two drafts of one request have cosine ~0.8.
  * Zipf-skewed router bias: ``b_e = s * (mean_r ln r - ln r_e)`` with
    ``r`` a seeded permutation of 1..E, so with no token signal the router's
    probabilities fall off as rank^-s.
  * bf16 tensors are drawn in float32 and rounded to nearest-even once, here;
    both sides consume the same bits.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "LayerConfig",
    "CONFIGS",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "make_layer",
    "make_hidden",
    "make_router",
    "make_expert_weights",
    "make_logits",
]

# Order in which per-tensor random streams are spawned from the seed.
_STREAMS = ("w_g", "bias_perm", "request_means", "token_noise", "gate", "up", "down")


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and input distribution of one MoE layer workload."""

    name: str
    d: int
    E: int
    k: int
    I: int
    dtype: str  # "bf16" or "f32"
    zipf_s: float
    batches: Sequence[int]
    hidden: str  # "iid", "requests", "drafts"
    n_requests: int = 16
    drafts_per_request: int = 4
    request_mean_std: float = 0.5
    token_noise_std: float = 1.0
    expert_std: float = 0.02
    oea_k0: Sequence[int] = ()
    budget_m: Sequence[int] = ()

    @property
    def bytes_per_weight(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert's gate, up and down matrices."""
        return 3 * self.d * self.I * self.bytes_per_weight


CONFIGS: Dict[str, LayerConfig] = {
    "tiny_f32": LayerConfig(
        name="tiny_f32", d=256, E=16, k=4, I=128, dtype="f32", zipf_s=1.2,
        batches=(4,), hidden="iid", oea_k0=(2,), budget_m=(4, 8)),
    "lynx_bf16": LayerConfig(
        name="lynx_bf16", d=2048, E=64, k=8, I=1408, dtype="bf16", zipf_s=1.1,
        batches=(16,), hidden="iid", oea_k0=(2, 4), budget_m=(24, 32)),
    "qwen3_30b_bf16": LayerConfig(
        name="qwen3_30b_bf16", d=2048, E=128, k=8, I=768, dtype="bf16", zipf_s=1.2,
        batches=(1, 4, 8, 16, 32), hidden="requests",
        oea_k0=(1, 2, 3, 4, 5, 6, 7, 8), budget_m=(24, 32, 48, 64)),
    "qwen3_235b_bf16": LayerConfig(
        name="qwen3_235b_bf16", d=4096, E=128, k=8, I=1536, dtype="bf16", zipf_s=1.2,
        batches=(1, 16, 64), hidden="requests", oea_k0=(4,), budget_m=(48,)),
    "specdec_bf16": LayerConfig(
        name="specdec_bf16", d=2048, E=128, k=8, I=768, dtype="bf16", zipf_s=1.2,
        batches=(64,), hidden="drafts", n_requests=16, drafts_per_request=4,
        request_mean_std=float(np.sqrt(0.8)), token_noise_std=float(np.sqrt(0.2)),
        oea_k0=(2, 4), budget_m=(32, 48, 64)),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits.

    Inputs must be finite. The result is a uint16 array of the same shape.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int) -> Dict[str, np.random.SeedSequence]:
    return dict(zip(_STREAMS, np.random.SeedSequence(seed).spawn(len(_STREAMS))))


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def _request_of_token(cfg: LayerConfig, B: int) -> np.ndarray:
    if cfg.hidden == "requests":
        return np.arange(B) % cfg.n_requests
    if cfg.hidden == "drafts":
        return np.arange(B) // cfg.drafts_per_request
    raise ValueError(cfg.hidden)


def make_hidden(cfg: LayerConfig, B: int, seed: int = 0) -> np.ndarray:
    """Hidden states x[B, d] (bf16 bits or float32).

    Token t's noise is the t-th row of one stream, so x for a batch B1 < B2 is
    a prefix of x for B2.
    """
    st = _streams(seed)
    noise = _rng(st["token_noise"]).standard_normal((B, cfg.d), dtype=np.float32)
    if cfg.hidden == "iid":
        x = noise
    else:
        n_req = int(_request_of_token(cfg, B).max()) + 1 if B > 0 else 0
        n_req = max(n_req, cfg.n_requests)
        means = _rng(st["request_means"]).standard_normal((n_req, cfg.d), dtype=np.float32)
        means *= np.float32(cfg.request_mean_std)
        x = means[_request_of_token(cfg, B)] + noise * np.float32(cfg.token_noise_std)
    return _store(x, cfg.dtype)


def make_router(cfg: LayerConfig, seed: int = 0, bias: bool = True):
    """Router weight W_g[d, E] (bf16 bits or float32) and float32 bias[E] (or None)."""
    st = _streams(seed)
    w = _rng(st["w_g"]).standard_normal((cfg.d, cfg.E), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(cfg.d))
    b = None
    if bias:
        r = _rng(st["bias_perm"]).permutation(cfg.E).astype(np.float64) + 1.0
        lr = np.log(r)
        b = (cfg.zipf_s * (lr.mean() - lr)).astype(np.float32)
    return _store(w, cfg.dtype), b


def _expert_block(args):
    ss, shape, std, dtype = args
    a = _rng(ss).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return _store(a, dtype)


def make_expert_weights(cfg: LayerConfig, seed: int = 0, experts: Optional[Sequence[int]] = None,
                        threads: Optional[int] = None):
    """Expert gate G[E,d,I], up U[E,d,I] and down D[E,I,d].

    Every expert of every matrix has its own stream, so a subset of experts
    (``experts``) is drawn bit-identically to the same experts of the full
    tensors; the result then has len(experts) leading rows in that order.
    """
    st = _streams(seed)
    ids = list(range(cfg.E)) if experts is None else [int(e) for e in experts]
    out = {}
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        for name, shape in (("gate", (cfg.d, cfg.I)), ("up", (cfg.d, cfg.I)), ("down", (cfg.I, cfg.d))):
            kids = st[name].spawn(cfg.E)
            jobs = [(kids[e], shape, cfg.expert_std, cfg.dtype) for e in ids]
            dt = np.uint16 if cfg.dtype == "bf16" else np.float32
            arr = np.empty((len(ids),) + shape, dtype=dt)
            for i, blk in enumerate(ex.map(_expert_block, jobs)):
                arr[i] = blk
            out[name] = arr
    return out["gate"], out["up"], out["down"]


def make_layer(cfg: LayerConfig, B: int, seed: int = 0, bias: bool = True,
               experts: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """All inputs of one layer call: x, w_g, bias, w_gate, w_up, w_down."""
    x = make_hidden(cfg, B, seed)
    w_g, b = make_router(cfg, seed, bias)
    g, u, dn = make_expert_weights(cfg, seed, experts)
    return {"x": x, "w_g": w_g, "bias": b, "w_gate": g, "w_up": u, "w_down": dn}


def make_logits(B: int, E: int, seed: int = 0, kind: str = "normal") -> np.ndarray:
    """Float32 logits[B, E] for exercising selection on its own.

    kinds: ``normal`` (iid N(0,1) plus a Zipf-like skew), ``ties`` (values on a
    coarse grid of 8 levels so many logits tie exactly, with some -0.0/+0.0
    pairs), ``flat`` (all equal).
    """
    rng = _rng(np.random.SeedSequence([seed, B, E, 0x5E1EC7]))
    if kind == "normal":
        r = rng.permutation(E).astype(np.float64) + 1.0
        skew = 1.2 * (np.log(r).mean() - np.log(r))
        return (rng.standard_normal((B, E)) + skew[None, :]).astype(np.float32)
    if kind == "ties":
        L = (rng.integers(-4, 4, size=(B, E)).astype(np.float32) * np.float32(0.5))
        zero = L == 0
        flip = rng.random((B, E)) < 0.5
        L[zero & flip] = np.float32(-0.0)
        return L
    if kind == "flat":
        return np.zeros((B, E), dtype=np.float32)
    raise ValueError(kind)
