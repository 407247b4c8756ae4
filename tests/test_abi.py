"""The C ABI: the library loads, exports every function the header declares,
and rejects bad arguments with the documented status before any HIP call.

These run without a GPU: every call below fails validation on the host, so
no kernel is launched and the fake device addresses are never touched.
"""
import ctypes
import os
import re

import pytest

from aware_expert_routing_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_decode.h")

A = 0x10000  # a 256-byte-aligned fake device address, never dereferenced


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    names = ["MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP",
             "MOE_ERR_RESIDENCY", "MOE_ERR_SYNC_TIMEOUT", "MOE_ERR_SCRATCH"]
    for s, name in enumerate(names):
        assert L.status_string(s).startswith(name)
        assert getattr(L, name) == s
    assert "unknown" in L.status_string(99)


def test_header_status_codes_match_binding():
    src = open(HEADER).read()
    for name, val in re.findall(r"\b(MOE_ERR_[A-Z_]+|MOE_OK) = (\d+)", src):
        assert getattr(L, name) == int(val), name
    assert int(re.search(r"#define MOE_WS_STATUS_BYTES (\d+)", src).group(1)) == L.MOE_WS_STATUS_BYTES
    m = re.search(r"#define MOE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert int(m.group(1)) << int(m.group(2)) == L.MOE_STATIC_SCRATCH_BYTES


def _layer_static(lib, **kw):
    a = dict(x=A, w_g=A, bias=None, wg=A, wu=A, wd=A, dt=L.MOE_BF16, B=16, d=2048, E=128, I=768,
             pol=L.Policy(L.MOE_POLICY_TOPK, 8, 0, 0), logits=A, r=_routing(), y=A, s=None)
    a.update(kw)
    r = a["r"]
    return lib.moe_layer_decode_static(a["x"], a["w_g"], a["bias"], a["wg"], a["wu"], a["wd"], a["dt"],
                                       a["B"], a["d"], a["E"], a["I"], a["pol"], a["logits"],
                                       ctypes.byref(r) if r is not None else None, a["y"], a["s"])


def test_static_layer_refuses_sizes_beyond_its_scratch(lib):
    """moe_layer_decode_static refuses, before any HIP call, sizes whose
    workspace would not fit its static scratch (the Qwen3-235B-shaped layer
    at B = 64 needs about 59 MB), and checks its arguments like
    moe_layer_decode."""
    assert lib.moe_workspace_bytes(64, 4096, 128, 1536, 8, L.MOE_BF16) > L.MOE_STATIC_SCRATCH_BYTES
    assert _layer_static(lib, B=64, d=4096, I=1536) == L.MOE_ERR_SCRATCH
    assert lib.moe_workspace_bytes(64, 2048, 128, 768, 8, L.MOE_BF16) <= L.MOE_STATIC_SCRATCH_BYTES
    assert _layer_static(lib, x=None) == L.MOE_ERR_INVALID_ARG
    assert _layer_static(lib, r=None) == L.MOE_ERR_INVALID_ARG
    assert _layer_static(lib, B=300) == L.MOE_ERR_UNSUPPORTED
    assert _layer_static(lib, pol=L.Policy(L.MOE_POLICY_OEA, 8, 0, 0)) == L.MOE_ERR_INVALID_ARG


def test_workspace_check_reads_the_status_word(lib):
    """A zero-filled workspace head is clean; the status word the expert FFN
    sets when a grid-wide wait gives up (byte 256, written here from the
    host) is reported as MOE_ERR_SYNC_TIMEOUT; other words (barrier count,
    release word, counters) do not matter; short or null buffers are
    rejected."""
    head = bytearray(L.MOE_WS_STATUS_BYTES)
    assert L.workspace_status(bytes(head)) == L.MOE_OK
    head[0:4] = (7).to_bytes(4, "little")      # arrival count mid-launch
    head[128:132] = (99).to_bytes(4, "little")  # release word (only grows)
    head[384:388] = (3).to_bytes(4, "little")   # router + selection counter
    assert L.workspace_status(bytes(head)) == L.MOE_OK
    head[256:260] = (1).to_bytes(4, "little")
    assert L.workspace_status(bytes(head)) == L.MOE_ERR_SYNC_TIMEOUT
    head[256:260] = (0x100).to_bytes(4, "little")  # any bit of the word
    assert L.workspace_status(bytes(head)) == L.MOE_ERR_SYNC_TIMEOUT
    assert L.workspace_status(bytes(head[:L.MOE_WS_STATUS_BYTES - 1])) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_check(None, L.MOE_WS_STATUS_BYTES) == L.MOE_ERR_INVALID_ARG


def test_workspace_bytes_envelope(lib):
    f = lib.moe_workspace_bytes
    assert f(16, 2048, 128, 768, 8, L.MOE_BF16) > 0
    assert f(4, 256, 16, 128, 4, L.MOE_F32) > 0
    assert f(0, 2048, 128, 768, 8, L.MOE_BF16) == 0       # B < 1
    assert f(257, 2048, 128, 768, 8, L.MOE_BF16) == 0     # B > 256
    assert f(16, 2048, 257, 768, 8, L.MOE_BF16) == 0      # E > 256
    assert f(16, 2047, 128, 768, 8, L.MOE_BF16) == 0      # d % 8
    assert f(16, 2048, 128, 770, 8, L.MOE_BF16) == 0      # I % 8
    assert f(16, 2048, 128, 768, 17, L.MOE_BF16) == 0     # k > 16
    assert f(16, 2048, 4, 768, 8, L.MOE_BF16) == 0        # k > E
    assert f(16, 2048, 128, 768, 8, 7) == 0               # dtype
    # grows with the batch
    assert f(64, 2048, 128, 768, 8, L.MOE_BF16) > f(16, 2048, 128, 768, 8, L.MOE_BF16)


def _routing(mass=True):
    return L.RoutingC(*([A] * 7 + [A if mass else None]))


def _layer(lib, **kw):
    a = dict(x=A, w_g=A, bias=None, wg=A, wu=A, wd=A, dt=L.MOE_BF16, B=16, d=2048, E=128, I=768,
             pol=L.Policy(L.MOE_POLICY_TOPK, 8, 0, 0), logits=A, r=_routing(), y=A, ws=A,
             wsb=1 << 40, s=None)
    a.update(kw)
    r = a["r"]
    return lib.moe_layer_decode(a["x"], a["w_g"], a["bias"], a["wg"], a["wu"], a["wd"], a["dt"],
                                a["B"], a["d"], a["E"], a["I"], a["pol"], a["logits"],
                                ctypes.byref(r) if r is not None else None, a["y"], a["ws"],
                                a["wsb"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), L.MOE_ERR_INVALID_ARG),
    (dict(x=A + 8), L.MOE_ERR_INVALID_ARG),              # not 16-byte aligned
    (dict(wd=None), L.MOE_ERR_INVALID_ARG),
    (dict(y=A + 4), L.MOE_ERR_INVALID_ARG),
    (dict(logits=None), L.MOE_ERR_INVALID_ARG),
    (dict(bias=A + 2), L.MOE_ERR_INVALID_ARG),
    (dict(r=None), L.MOE_ERR_INVALID_ARG),
    (dict(dt=5), L.MOE_ERR_INVALID_ARG),
    (dict(B=0), L.MOE_ERR_INVALID_ARG),
    (dict(B=257), L.MOE_ERR_UNSUPPORTED),
    (dict(E=300), L.MOE_ERR_UNSUPPORTED),
    (dict(d=2044), L.MOE_ERR_UNSUPPORTED),
    (dict(I=4), L.MOE_ERR_UNSUPPORTED),
    (dict(pol=L.Policy(L.MOE_POLICY_TOPK, 0, 0, 0)), L.MOE_ERR_INVALID_ARG),
    (dict(pol=L.Policy(L.MOE_POLICY_TOPK, 129, 0, 0)), L.MOE_ERR_INVALID_ARG),  # k > E
    (dict(pol=L.Policy(L.MOE_POLICY_TOPK, 17, 0, 0)), L.MOE_ERR_UNSUPPORTED),
    (dict(pol=L.Policy(L.MOE_POLICY_OEA, 8, 0, 0)), L.MOE_ERR_INVALID_ARG),     # k0 < 1
    (dict(pol=L.Policy(L.MOE_POLICY_OEA, 8, 9, 0)), L.MOE_ERR_INVALID_ARG),     # k0 > k
    (dict(pol=L.Policy(L.MOE_POLICY_BUDGET, 8, 0, 0)), L.MOE_ERR_INVALID_ARG),  # m < 1
    (dict(pol=L.Policy(L.MOE_POLICY_BUDGET, 8, 0, 129)), L.MOE_ERR_INVALID_ARG),  # m > E
    (dict(pol=L.Policy(L.MOE_POLICY_BUDGET, 8, 0, 32), r=_routing(mass=False)), L.MOE_ERR_INVALID_ARG),
    (dict(pol=L.Policy(L.MOE_POLICY_GREEDY, 8, 0, 0)), L.MOE_ERR_INVALID_ARG),  # m < 1
    (dict(pol=L.Policy(L.MOE_POLICY_GREEDY, 8, 0, 129)), L.MOE_ERR_INVALID_ARG),  # m > E
    (dict(pol=L.Policy(L.MOE_POLICY_HIER, 8, 4, 0, 4)), L.MOE_ERR_INVALID_ARG),   # m < 1
    (dict(pol=L.Policy(L.MOE_POLICY_HIER, 8, 0, 32, 4)), L.MOE_ERR_INVALID_ARG),  # m_r < 1
    (dict(pol=L.Policy(L.MOE_POLICY_HIER, 8, 33, 32, 4)), L.MOE_ERR_INVALID_ARG),  # m_r > m
    (dict(pol=L.Policy(L.MOE_POLICY_HIER, 8, 8, 32, 0)), L.MOE_ERR_INVALID_ARG),  # g < 1
    (dict(pol=L.Policy(L.MOE_POLICY_HIER, 8, 8, 129, 4)), L.MOE_ERR_INVALID_ARG),  # m > E
    (dict(pol=L.Policy(L.MOE_POLICY_LYNX, 8, 0, 7)), L.MOE_ERR_INVALID_ARG),      # m < k
    (dict(pol=L.Policy(L.MOE_POLICY_LYNX, 8, 0, 129)), L.MOE_ERR_INVALID_ARG),    # m > E
    (dict(pol=L.Policy(6, 8, 0, 32)), L.MOE_ERR_INVALID_ARG),                     # unknown kind
    (dict(pol=L.Policy(L.MOE_POLICY_HIER, 8, 8, 32, 4), r=_routing(mass=False)), L.MOE_ERR_INVALID_ARG),
    (dict(pol=L.Policy(7, 8, 0, 0)), L.MOE_ERR_INVALID_ARG),
    (dict(ws=None), L.MOE_ERR_WORKSPACE),
    (dict(ws=A + 16), L.MOE_ERR_WORKSPACE),             # not 256-byte aligned
    (dict(wsb=1024), L.MOE_ERR_WORKSPACE),
])
def test_layer_validation(lib, kw, status):
    assert _layer(lib, **kw) == status


def test_workspace_exactly_required_minus_one(lib):
    need = lib.moe_workspace_bytes(16, 2048, 128, 768, 8, L.MOE_BF16)
    assert _layer(lib, wsb=need - 1) == L.MOE_ERR_WORKSPACE


def test_route_validation(lib):
    f = lib.moe_route
    ok = dict(x=A, w=A, b=None, dt=L.MOE_BF16, B=16, d=2048, E=128, lg=A, ws=A, wsb=1 << 30, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["w"], a["b"], a["dt"], a["B"], a["d"], a["E"], a["lg"], a["ws"], a["wsb"], a["s"])

    assert call(x=None) == L.MOE_ERR_INVALID_ARG
    assert call(w=A + 2) == L.MOE_ERR_INVALID_ARG
    assert call(lg=None) == L.MOE_ERR_INVALID_ARG
    assert call(E=0) == L.MOE_ERR_INVALID_ARG
    assert call(d=12) == L.MOE_ERR_UNSUPPORTED
    assert call(wsb=16) == L.MOE_ERR_WORKSPACE
    assert call(ws=None) == L.MOE_ERR_WORKSPACE


def test_select_validation(lib):
    f = lib.moe_select

    def call(lg=A, B=16, E=128, pol=None, r="default"):
        pol = pol or L.Policy(L.MOE_POLICY_OEA, 8, 2, 0)
        rr = _routing() if r == "default" else r
        return f(lg, B, E, pol, ctypes.byref(rr) if rr is not None else None, None)

    assert call(lg=None) == L.MOE_ERR_INVALID_ARG
    assert call(lg=A + 1) == L.MOE_ERR_INVALID_ARG
    assert call(B=0) == L.MOE_ERR_INVALID_ARG
    assert call(B=300) == L.MOE_ERR_UNSUPPORTED
    assert call(pol=L.Policy(L.MOE_POLICY_OEA, 8, 0, 0)) == L.MOE_ERR_INVALID_ARG
    assert call(r=None) == L.MOE_ERR_INVALID_ARG
    bad = _routing()
    bad.pair_slot = None
    assert call(r=bad) == L.MOE_ERR_INVALID_ARG
    bad = _routing()
    bad.topk_w = A + 2
    assert call(r=bad) == L.MOE_ERR_INVALID_ARG
    assert call(pol=L.Policy(L.MOE_POLICY_BUDGET, 8, 0, 16), r=_routing(mass=False)) == L.MOE_ERR_INVALID_ARG
    assert call(pol=L.Policy(L.MOE_POLICY_GREEDY, 8, 0, 0)) == L.MOE_ERR_INVALID_ARG
    # GREEDY does not use batch_mass.
    assert call(pol=L.Policy(L.MOE_POLICY_GREEDY, 8, 0, 0), r=_routing(mass=False)) == L.MOE_ERR_INVALID_ARG


def test_ffn_validation(lib):
    f = lib.moe_expert_ffn
    r = _routing()

    def call(**kw):
        a = dict(x=A, g=A, u=A, dn=A, dt=L.MOE_BF16, B=16, d=2048, E=128, I=768, k=8, y=A, ws=A,
                 wsb=1 << 40)
        a.update(kw)
        return f(a["x"], a["g"], a["u"], a["dn"], a["dt"], a["B"], a["d"], a["E"], a["I"], a["k"],
                 ctypes.byref(r), a["y"], a["ws"], a["wsb"], None)

    assert call(g=None) == L.MOE_ERR_INVALID_ARG
    assert call(u=A + 8) == L.MOE_ERR_INVALID_ARG
    assert call(k=0) == L.MOE_ERR_INVALID_ARG
    assert call(k=200) == L.MOE_ERR_INVALID_ARG
    assert call(I=12) == L.MOE_ERR_UNSUPPORTED
    assert call(wsb=100) == L.MOE_ERR_WORKSPACE


def test_read_stream_validation(lib):
    st = L.MOE_ERR_INVALID_ARG
    assert lib.moe_read_stream(None, 1024, A, None) == st
    assert lib.moe_read_stream(A + 8, 1024, A, None) == st   # misaligned source
    assert lib.moe_read_stream(A, 0, A, None) == st          # empty
    assert lib.moe_read_stream(A, 1000, A, None) == st       # not a multiple of 16
    assert lib.moe_read_stream(A, 1024, None, None) == st    # no output
