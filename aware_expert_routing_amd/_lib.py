"""ctypes binding of libmoe_decode.so (include/moe_decode.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the shared library. Functions take torch tensors for device memory and a
torch stream; they check dtype/device/shape/contiguity on the host and raise
``MoeError`` with the library's status string when a call fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_decode.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_ERR_RESIDENCY = 5
MOE_ERR_SYNC_TIMEOUT = 6
MOE_ERR_SCRATCH = 7
MOE_WS_STATUS_BYTES = 512
MOE_STATIC_SCRATCH_BYTES = 32 << 20

MOE_F32 = 0
MOE_BF16 = 1

MOE_POLICY_TOPK = 0
MOE_POLICY_OEA = 1
MOE_POLICY_BUDGET = 2
MOE_POLICY_GREEDY = 3
MOE_POLICY_HIER = 4
MOE_POLICY_LYNX = 5

EXPORTS = ("moe_workspace_bytes", "moe_workspace_check", "moe_route", "moe_select",
           "moe_expert_ffn", "moe_layer_decode", "moe_layer_decode_static", "moe_status_string",
           "moe_read_stream")


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Policy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("k", ctypes.c_int32), ("k0", ctypes.c_int32),
                ("m", ctypes.c_int32), ("g", ctypes.c_int32)]


_ROUTING_FIELDS = ("topk_ids", "topk_w", "n_active", "active_experts", "expert_offsets",
                   "pair_token", "pair_slot", "batch_mass")


class RoutingC(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in _ROUTING_FIELDS]


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the shared library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m aware_expert_routing_amd.build`")
    lib = ctypes.CDLL(p)
    vp, c_int, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_workspace_bytes.restype = sz
    lib.moe_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    lib.moe_route.restype = c_int
    lib.moe_route.argtypes = [vp, vp, vp, c_int, c_int, c_int, c_int, vp, vp, sz, vp]
    lib.moe_select.restype = c_int
    lib.moe_select.argtypes = [vp, c_int, c_int, Policy, ctypes.POINTER(RoutingC), vp]
    lib.moe_expert_ffn.restype = c_int
    lib.moe_expert_ffn.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                   ctypes.POINTER(RoutingC), vp, vp, sz, vp]
    lib.moe_layer_decode.restype = c_int
    lib.moe_layer_decode.argtypes = [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                     Policy, vp, ctypes.POINTER(RoutingC), vp, vp, sz, vp]
    lib.moe_layer_decode_static.restype = c_int
    lib.moe_layer_decode_static.argtypes = [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                            Policy, vp, ctypes.POINTER(RoutingC), vp, vp]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [c_int]
    lib.moe_workspace_check.restype = c_int
    lib.moe_workspace_check.argtypes = [vp, sz]
    lib.moe_read_stream.restype = c_int
    lib.moe_read_stream.argtypes = [vp, sz, vp, vp]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, status_string(status))


def make_policy(kind: str, k: int, k0: int = 0, m: int = 0, g: int = 0) -> Policy:
    """kind: topk | oea (k0) | budget (m) | greedy (m) | hier (m, k0 = request
    budget m_r, g = tokens per request) | lynx (m, the critical-set size)."""
    kinds = {"topk": MOE_POLICY_TOPK, "oea": MOE_POLICY_OEA, "budget": MOE_POLICY_BUDGET,
             "greedy": MOE_POLICY_GREEDY, "hier": MOE_POLICY_HIER, "lynx": MOE_POLICY_LYNX}
    if kind not in kinds:
        raise ValueError(f"unknown policy {kind!r}")
    return Policy(kinds[kind], int(k), int(k0), int(m), int(g))


# ----------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Routing:
    """Device buffers of one selection (the fields of moe_routing_t)."""

    def __init__(self, B: int, E: int, k: int, device="cuda", with_mass: bool = True):
        torch = _torch()
        i32 = dict(dtype=torch.int32, device=device)
        self.B, self.E, self.k = B, E, k
        self.topk_ids = torch.empty((B, k), **i32)
        self.topk_w = torch.empty((B, k), dtype=torch.float32, device=device)
        self.n_active = torch.empty((1,), **i32)
        self.active_experts = torch.empty((E,), **i32)
        self.expert_offsets = torch.empty((E + 1,), **i32)
        self.pair_token = torch.empty((B * k,), **i32)
        self.pair_slot = torch.empty((B * k,), **i32)
        self.batch_mass = torch.empty((E,), dtype=torch.float32, device=device) if with_mass else None

    def c_struct(self) -> RoutingC:
        return RoutingC(*[_ptr(getattr(self, f)) for f in _ROUTING_FIELDS])


def moe_workspace_bytes(B: int, d: int, E: int, I: int, k: int, dtype) -> int:
    torch = _torch()
    dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load().moe_workspace_bytes(B, d, E, I, k, dt))


def alloc_workspace(B: int, d: int, E: int, I: int, k: int, dtype, device="cuda"):
    torch = _torch()
    n = moe_workspace_bytes(B, d, E, I, k, dtype)
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, status_string(MOE_ERR_UNSUPPORTED))
    # Zero-filled once: the expert FFN keeps its grid-barrier words here.
    return torch.zeros((n,), dtype=torch.uint8, device=device)


def workspace_status(workspace_head: bytes) -> int:
    """moe_workspace_check on a host copy of a workspace's first
    MOE_WS_STATUS_BYTES bytes; returns the status code."""
    buf = ctypes.create_string_buffer(bytes(workspace_head), len(workspace_head))
    return int(load().moe_workspace_check(ctypes.cast(buf, ctypes.c_void_p), len(workspace_head)))


def check_workspace(workspace) -> None:
    """Copies the status bytes of a device workspace (waiting for the
    current stream) and raises MoeError if a grid-wide wait of the expert FFN
    gave up in any call since the workspace was zero-filled."""
    head = workspace[:MOE_WS_STATUS_BYTES].cpu().numpy().tobytes()
    _check(workspace_status(head))


def moe_route(x, w_g, bias, logits, workspace, stream=None):
    B, d = x.shape
    E = w_g.shape[1]
    if w_g.shape[0] != d or tuple(logits.shape) != (B, E) or w_g.dtype != x.dtype:
        raise ValueError("shape/dtype mismatch")
    _check(load().moe_route(_ptr(x), _ptr(w_g), _ptr(bias), _dt(x), B, d, E, _ptr(logits),
                            _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_select(logits, policy: Policy, routing: Routing, stream=None):
    B, E = logits.shape
    if (routing.B, routing.E, routing.k) != (B, E, policy.k):
        raise ValueError("routing buffers do not match B, E, k")
    r = routing.c_struct()
    _check(load().moe_select(_ptr(logits), B, E, policy, ctypes.byref(r), _stream(stream)))


def moe_read_stream(src, out, stream=None):
    """Read-only scan of the whole of `src` (a contiguous device tensor whose
    byte size is a multiple of 16); out: int32/uint32 device tensor of 1024
    words receiving each workgroup's XOR. A measurement utility."""
    _check(load().moe_read_stream(_ptr(src), src.numel() * src.element_size(), _ptr(out),
                                  _stream(stream)))


def moe_expert_ffn(x, w_gate, w_up, w_down, routing: Routing, y, workspace, stream=None, lib=None):
    B, d = x.shape
    E, d2, I = w_gate.shape
    if d2 != d or tuple(w_up.shape) != (E, d, I) or tuple(w_down.shape) != (E, I, d):
        raise ValueError("expert weight shapes must be [E,d,I], [E,d,I], [E,I,d]")
    if tuple(y.shape) != (B, d) or y.dtype != x.dtype:
        raise ValueError("y must be [B,d] in the input dtype")
    r = routing.c_struct()
    _check((lib or load()).moe_expert_ffn(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _dt(x), B, d, E,
                                 I, routing.k, ctypes.byref(r), _ptr(y), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))


def moe_layer_decode(x, w_g, bias, w_gate, w_up, w_down, policy: Policy, logits,
                     routing: Routing, y, workspace, stream=None):
    B, d = x.shape
    E, d2, I = w_gate.shape
    if d2 != d or tuple(w_g.shape) != (d, E) or tuple(w_up.shape) != (E, d, I) \
            or tuple(w_down.shape) != (E, I, d) or tuple(y.shape) != (B, d):
        raise ValueError("shape mismatch")
    if tuple(logits.shape) != (B, E) or (routing.B, routing.E, routing.k) != (B, E, policy.k):
        raise ValueError("logits/routing buffers do not match B, E, k")
    r = routing.c_struct()
    _check(load().moe_layer_decode(_ptr(x), _ptr(w_g), _ptr(bias), _ptr(w_gate), _ptr(w_up),
                                   _ptr(w_down), _dt(x), B, d, E, I, policy, _ptr(logits),
                                   ctypes.byref(r), _ptr(y), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))


def moe_layer_decode_static(x, w_g, bias, w_gate, w_up, w_down, policy: Policy, logits,
                            routing: Routing, y, stream=None):
    """moe_layer_decode with the library's static device scratch instead of a
    workspace (allocates nothing); calls on one device must not overlap."""
    B, d = x.shape
    E, d2, I = w_gate.shape
    if d2 != d or tuple(w_g.shape) != (d, E) or tuple(w_up.shape) != (E, d, I) \
            or tuple(w_down.shape) != (E, I, d) or tuple(y.shape) != (B, d):
        raise ValueError("shape mismatch")
    if tuple(logits.shape) != (B, E) or (routing.B, routing.E, routing.k) != (B, E, policy.k):
        raise ValueError("logits/routing buffers do not match B, E, k")
    r = routing.c_struct()
    _check(load().moe_layer_decode_static(_ptr(x), _ptr(w_g), _ptr(bias), _ptr(w_gate), _ptr(w_up),
                                          _ptr(w_down), _dt(x), B, d, E, I, policy, _ptr(logits),
                                          ctypes.byref(r), _ptr(y), _stream(stream)))
