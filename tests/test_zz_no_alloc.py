"""moe_layer_decode_static (no workspace, static device scratch) against
moe_layer_decode (caller workspace) through the C ABI: two calls in a row,
the second with a smaller batch, each bit-identical to the workspace entry
point on the same inputs (same kernels, same order of arithmetic)."""
import numpy as np
import pytest
import torch

from aware_expert_routing_amd import _lib as L
from aware_expert_routing_amd.workloads import CONFIGS, make_layer
from gpu_helpers import routing_numpy, to_dev

pytestmark = pytest.mark.gpu


def _run(fn_static, cfg, dev, B, pol, k0, m):
    x = dev["x"][:B].contiguous()
    policy = L.make_policy(pol, cfg.k, k0, m)
    r = L.Routing(B, cfg.E, cfg.k)
    lg = torch.empty((B, cfg.E), dtype=torch.float32, device="cuda")
    y = torch.empty((B, cfg.d), dtype=torch.bfloat16, device="cuda")
    args = (x, dev["w_g"], dev["bias"], dev["w_gate"], dev["w_up"], dev["w_down"], policy, lg, r, y)
    if fn_static:
        L.moe_layer_decode_static(*args)
    else:
        ws = L.alloc_workspace(B, cfg.d, cfg.E, cfg.I, cfg.k, torch.bfloat16)
        L.moe_layer_decode(*args, ws)
        torch.cuda.synchronize()
        L.check_workspace(ws)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), routing_numpy(r), y.clone()


def test_static_scratch_layer_matches_workspace_layer():
    cfg = CONFIGS["qwen3_30b_bf16"]
    inp = make_layer(cfg, 32)
    dev = {k: to_dev(v, cfg.dtype) for k, v in inp.items()}
    # Two calls in a row on the same static scratch, the second smaller, then
    # a third larger one again.
    for B, pol, k0, m in ((32, "oea", 4, 0), (4, "budget", 0, 24), (16, "topk", 0, 0)):
        print(f"\n[case] static scratch B={B} {pol}", flush=True)
        Ls, rs, ys = _run(True, cfg, dev, B, pol, k0, m)
        Lw, rw, yw = _run(False, cfg, dev, B, pol, k0, m)
        assert np.array_equal(Ls, Lw), f"B={B} {pol}: logits"
        for key in ("ids", "w", "n_active", "active", "offsets", "pair_token", "pair_slot"):
            assert np.array_equal(np.asarray(rs[key]), np.asarray(rw[key])), f"B={B} {pol}: {key}"
        assert torch.equal(ys, yw), f"B={B} {pol}: y"
