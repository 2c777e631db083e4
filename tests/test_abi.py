"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import re

import pytest

import moe_decode_sigmoid_amd as moe
from tests.conftest import ROOT

HEADER = ROOT / "include" / "moe_decode.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["moe_decode_route", "moe_decode_forward", "moe_decode_forward_timed",
              "moe_prefill_forward", "moe_nvfp4_gemv", "moe_decode_forward_ex",
              "moe_prefill_forward_ex", "moe_decode_stack_forward",
              "moe_decode_chain_forward", "moe_workspace_status",
              "moe_general_workspace_layout",
              "moe_nvfp4_dequant", "moe_workspace_bytes", "moe_status_string",
              "moe_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in the header but not exported"


def test_status_strings_and_version():
    assert moe.abi_version() == 1
    assert moe.status_string(moe.MOE_OK) == "MOE_OK"
    assert moe.status_string(moe.MOE_ERR_UNSUPPORTED) == "MOE_ERR_UNSUPPORTED"
    assert moe.status_string(-99) == "MOE_ERR_UNKNOWN"


def test_workspace_sizes():
    for B in range(1, 9):
        assert moe.moe_workspace_bytes(B) > 0
    assert moe.moe_workspace_bytes(9) == 0
    assert moe.moe_workspace_bytes(0) == 0
    S = moe.shape(moe.MOE_W_NVFP4, hidden=4100)
    assert moe.lib().moe_workspace_bytes(ctypes.byref(S), 1, 0) == 0
    S = moe.shape(moe.MOE_W_NVFP4, hidden=4096)                  # general decode path
    assert moe.lib().moe_workspace_bytes(ctypes.byref(S), 1, 0) > 0


# Fake, never-dereferenced device addresses: every call below must be refused
# by the argument checks, which run before any HIP call.
A = 0x7F0000000000          # 256-byte aligned
WS_BIG = 1 << 30


class _FakeExperts:
    def __init__(self, base, fmt="nvfp4"):
        self.w13 = base
        self.w2 = base + 0x100000
        if fmt == "nvfp4":
            self.w13_scale = base + 0x200000
            self.w2_scale = base + 0x300000
            self.glob = base + 0x400000


def _forward(S=None, x=A, B=1, router=A + 0x1000000, routed=None, shared=None, out=A + 0x2000000,
             ids=None, w=None, ws=A + 0x3000000, ws_bytes=WS_BIG, prefill=False):
    S = S or moe.shape()
    R = moe.experts_struct(routed or _FakeExperts(A + 0x4000000))
    Sh = moe.experts_struct(shared or _FakeExperts(A + 0x5000000))
    fn = moe.lib().moe_prefill_forward if prefill else moe.lib().moe_decode_forward
    return fn(ctypes.byref(S), x, B, router, ctypes.byref(R), ctypes.byref(Sh), out, ids, w, ws,
              ws_bytes, 0)


@pytest.mark.parametrize("prefill", [False, True])
def test_forward_argument_errors(prefill):
    E = moe
    if prefill and moe.moe_workspace_bytes(8192, prefill=True) == 0:
        pytest.skip("prefill path not built into this library")
    assert _forward(x=None, prefill=prefill) == E.MOE_ERR_INVALID_ARG
    assert _forward(router=None, prefill=prefill) == E.MOE_ERR_INVALID_ARG
    assert _forward(out=None, prefill=prefill) == E.MOE_ERR_INVALID_ARG
    assert _forward(B=0, prefill=prefill) == E.MOE_ERR_INVALID_ARG
    assert _forward(x=A + 8, prefill=prefill) == E.MOE_ERR_MISALIGNED
    assert _forward(out=A + 0x2000004, prefill=prefill) == E.MOE_ERR_MISALIGNED
    assert _forward(ws=A + 0x3000010, prefill=prefill) == E.MOE_ERR_MISALIGNED
    assert _forward(ws=None, prefill=prefill) == E.MOE_ERR_WORKSPACE
    assert _forward(ws_bytes=1024, prefill=prefill) == E.MOE_ERR_WORKSPACE
    assert _forward(out=A, prefill=prefill) == E.MOE_ERR_INVALID_ARG            # out aliases x
    assert _forward(out=A + 0x3000000 + 4096, prefill=prefill) == E.MOE_ERR_INVALID_ARG  # in ws
    bad = _FakeExperts(A + 0x4000000)
    bad.w2_scale = None
    assert _forward(routed=bad, prefill=prefill) == E.MOE_ERR_INVALID_ARG
    bf = _FakeExperts(A + 0x4000000)                     # BF16 sets carry no scales
    assert _forward(S=moe.shape(moe.MOE_W_BF16), routed=bf, prefill=prefill) == E.MOE_ERR_INVALID_ARG
    assert _forward(ids=A + 2, prefill=prefill) == E.MOE_ERR_MISALIGNED
    # shapes the general decode path serves: prefill refuses them; decode accepts
    # them and still checks the rest first (here: a workspace that is too small)
    for kw in [dict(hidden=4096), dict(inter=1024), dict(n_experts=384), dict(top_k=8),
               dict(n_shared=2), dict(n_experts=384, top_k=8, n_shared=0)]:
        got = _forward(S=moe.shape(**kw), prefill=prefill, ws_bytes=1024)
        assert got == (E.MOE_ERR_UNSUPPORTED if prefill else E.MOE_ERR_WORKSPACE), kw
    # outside every path
    for kw in [dict(hidden=4100), dict(inter=48), dict(n_experts=1024), dict(top_k=9),
               dict(n_shared=3), dict(n_experts=4, top_k=6), dict(hidden=16384)]:
        assert _forward(S=moe.shape(**kw), prefill=prefill) == E.MOE_ERR_UNSUPPORTED, kw
    assert _forward(S=moe.shape(7), prefill=prefill) == E.MOE_ERR_UNSUPPORTED


def test_timed_forward_needs_both_events_and_checks_like_forward():
    S = moe.shape()
    R = moe.experts_struct(_FakeExperts(A + 0x4000000))
    Sh = moe.experts_struct(_FakeExperts(A + 0x5000000))
    fn = moe.lib().moe_decode_forward_timed

    def call(ev0, ev1, x=A, B=1):
        return fn(ctypes.byref(S), x, B, A + 0x1000000, ctypes.byref(R), ctypes.byref(Sh),
                  A + 0x2000000, None, None, A + 0x3000000, WS_BIG, 0, ev0, ev1)
    assert call(None, None) == moe.MOE_ERR_INVALID_ARG
    assert call(A, None) == moe.MOE_ERR_INVALID_ARG
    assert call(A, A, x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(A, A, B=9) == moe.MOE_ERR_UNSUPPORTED


def test_gemv_argument_errors():
    fn = moe.lib().moe_nvfp4_gemv

    def call(x=A, B=1, K=2048, N=64, codes=A + 0x1000000, scales=A + 0x2000000,
             glob=A + 0x3000000, y=A + 0x4000000):
        return fn(x, B, K, N, codes, scales, glob, y, 0)
    E = moe
    assert call(x=None) == E.MOE_ERR_INVALID_ARG
    assert call(codes=None) == E.MOE_ERR_INVALID_ARG
    assert call(y=None) == E.MOE_ERR_INVALID_ARG
    assert call(glob=None) == E.MOE_ERR_INVALID_ARG
    assert call(x=A + 8) == E.MOE_ERR_MISALIGNED
    assert call(codes=A + 0x1000008) == E.MOE_ERR_MISALIGNED
    assert call(scales=A + 0x2000001) == E.MOE_ERR_MISALIGNED
    assert call(B=0) == E.MOE_ERR_INVALID_ARG
    assert call(N=0) == E.MOE_ERR_INVALID_ARG
    assert call(K=48) == E.MOE_ERR_INVALID_ARG                 # not a multiple of 32
    assert call(K=0) == E.MOE_ERR_INVALID_ARG
    assert call(B=9) == E.MOE_ERR_UNSUPPORTED
    assert call(K=16384) == E.MOE_ERR_UNSUPPORTED
    assert call(B=8, K=8192) == E.MOE_ERR_UNSUPPORTED          # x no longer fits LDS
    assert call(y=A + 64) == E.MOE_ERR_INVALID_ARG             # y overlaps x


@pytest.mark.parametrize("prefill", [False, True])
def test_fused_neighbour_argument_errors(prefill):
    """Every call here fails a check before any launch (none may pass them all:
    the pointers are fake)."""
    E = moe
    S = moe.shape()
    R = moe.experts_struct(_FakeExperts(A + 0x4000000))
    Sh = moe.experts_struct(_FakeExperts(A + 0x5000000))
    fn = moe.lib().moe_prefill_forward_ex if prefill else moe.lib().moe_decode_forward_ex
    X, OUT, WS = A, A + 0x2000000, A + 0x3000000
    NW, RES, XN = A + 0x50000000, A + 0x51000000, A + 0x52000000   # past the workspace

    def call(B=2, **f):
        F = moe.Fuse(f.get("norm_w"), f.get("eps", 1e-6), f.get("residual"), f.get("xn_out"))
        return fn(ctypes.byref(S), X, B, ctypes.byref(F), A + 0x1000000, ctypes.byref(R),
                  ctypes.byref(Sh), OUT, None, None, WS, WS_BIG, 0)
    assert call(norm_w=NW + 2) == E.MOE_ERR_MISALIGNED
    assert call(norm_w=NW, eps=0.0) == E.MOE_ERR_INVALID_ARG
    assert call(norm_w=NW, eps=-1.0) == E.MOE_ERR_INVALID_ARG
    assert call(norm_w=NW, eps=float("nan")) == E.MOE_ERR_INVALID_ARG
    assert call(norm_w=NW, eps=float("inf")) == E.MOE_ERR_INVALID_ARG
    assert call(norm_w=OUT + 64) == E.MOE_ERR_INVALID_ARG        # weight inside out
    assert call(residual=RES + 8) == E.MOE_ERR_MISALIGNED
    assert call(residual=OUT + 4096) == E.MOE_ERR_INVALID_ARG    # partly overlaps out
    assert call(residual=WS + 1024) == E.MOE_ERR_INVALID_ARG     # inside the workspace
    assert call(xn_out=XN) == E.MOE_ERR_INVALID_ARG              # needs the norm
    assert call(norm_w=NW, xn_out=XN + 4) == E.MOE_ERR_MISALIGNED
    assert call(norm_w=NW, xn_out=X + 16) == E.MOE_ERR_INVALID_ARG
    assert call(norm_w=NW, xn_out=OUT) == E.MOE_ERR_INVALID_ARG
    assert call(norm_w=NW, residual=RES, xn_out=RES + 4096) == E.MOE_ERR_INVALID_ARG
    # the layer's own checks still come first
    assert call(B=0, norm_w=NW) == E.MOE_ERR_INVALID_ARG
    if not prefill:
        assert call(B=9, norm_w=NW) == E.MOE_ERR_UNSUPPORTED


def test_general_shapes_workspace_and_expert_checks():
    """General decode shapes: workspace sizes, MXFP8 sets (scales, no global),
    a missing shared set only when the shape has none.  Every call below
    fails a check (fake pointers must never reach a launch)."""
    S = moe.shape(moe.MOE_W_MXFP8, n_experts=384, top_k=8, n_shared=0)
    L = moe.lib()
    need = L.moe_workspace_bytes(ctypes.byref(S), 8, 0)
    assert need > 0 and L.moe_workspace_bytes(ctypes.byref(S), 9, 0) == 0
    assert L.moe_workspace_bytes(ctypes.byref(S), 8, 1) == 0          # no general prefill
    assert moe.moe_workspace_bytes(1) == moe.moe_workspace_bytes(8)   # Flint: one size

    class MX:
        def __init__(self, base, glob=None):
            self.w13, self.w2 = base, base + 0x100000
            self.w13_scale, self.w2_scale, self.glob = base + 0x200000, base + 0x300000, glob
    R = moe.experts_struct(MX(A + 0x4000000))
    fn = L.moe_decode_forward

    def call(S=S, routed=R, shared=None, ws_bytes=need - 256, out=A + 0x2000000):
        return fn(ctypes.byref(S), A, 2, A + 0x1000000, ctypes.byref(routed),
                  None if shared is None else ctypes.byref(shared), out, None, None,
                  A + 0x3000000, ws_bytes, 0)
    assert call() == moe.MOE_ERR_WORKSPACE                 # shared NULL is fine with none
    assert call(routed=moe.experts_struct(MX(A + 0x4000000, glob=A))) == moe.MOE_ERR_INVALID_ARG
    bad = MX(A + 0x4000000)
    bad.w2_scale = None
    assert call(routed=moe.experts_struct(bad)) == moe.MOE_ERR_INVALID_ARG
    S2 = moe.shape(moe.MOE_W_MXFP8, n_shared=2)
    assert call(S=S2) == moe.MOE_ERR_INVALID_ARG            # two shared experts, set missing
    assert call(S=S2, shared=R, ws_bytes=1024) == moe.MOE_ERR_WORKSPACE
    # the fused-neighbour entry and the dequant probe stay Flint-only
    F = moe.Fuse(None, 1e-6, None, None)
    assert L.moe_decode_forward_ex(ctypes.byref(S), A, 2, ctypes.byref(F), A + 0x1000000,
                                   ctypes.byref(R), None, A + 0x2000000, None, None,
                                   A + 0x3000000, WS_BIG, 0) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_nvfp4_dequant(ctypes.byref(S), ctypes.byref(R), 0, 0, A, 0) == \
        moe.MOE_ERR_UNSUPPORTED


def test_stack_argument_errors():
    """Every call fails a host-side check (the layer table is a fake device
    address and must never be read)."""
    L = moe.lib()
    S = moe.shape()
    T = A + 0x6000000

    def call(S=S, n=4, layers=T, x=A, B=2, out=A + 0x2000000, ids=None, ws=A + 0x3000000,
             wsb=1024):
        return L.moe_decode_stack_forward(ctypes.byref(S), n, layers, x, B, out, ids, ws, wsb, 0)
    assert call() == moe.MOE_ERR_WORKSPACE
    assert call(n=0, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG
    assert call(layers=None, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG
    assert call(layers=T + 4, wsb=WS_BIG) == moe.MOE_ERR_MISALIGNED
    assert call(B=9, wsb=WS_BIG) == moe.MOE_ERR_UNSUPPORTED
    assert call(B=0, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG
    assert call(x=A + 8) == moe.MOE_ERR_MISALIGNED
    assert call(ids=A + 2) == moe.MOE_ERR_MISALIGNED
    assert call(out=A + 4096, ws=A + 0x50000000, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG  # x
    assert call(S=moe.shape(n_experts=384, top_k=8, n_shared=0), wsb=WS_BIG) == \
        moe.MOE_ERR_UNSUPPORTED


def test_chain_argument_errors():
    """The chained stack's host-side checks (fake addresses, never read)."""
    L = moe.lib()
    S = moe.shape()
    T = A + 0x6000000
    NW = A + 0x50000000

    def call(S=S, n=4, layers=T, x=A, B=2, nw=None, eps=1e-6, out=A + 0x2000000, ids=None,
             ws=A + 0x3000000, wsb=1024):
        return L.moe_decode_chain_forward(ctypes.byref(S), n, layers, x, B, nw, eps, out, ids, ws,
                                          wsb, 0)
    assert call() == moe.MOE_ERR_WORKSPACE
    assert call(n=0, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG
    assert call(layers=None, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG
    assert call(layers=T + 4, wsb=WS_BIG) == moe.MOE_ERR_MISALIGNED
    assert call(B=9, wsb=WS_BIG) == moe.MOE_ERR_UNSUPPORTED
    assert call(B=0, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG
    assert call(x=A + 8) == moe.MOE_ERR_MISALIGNED
    assert call(nw=NW + 2) == moe.MOE_ERR_MISALIGNED
    assert call(nw=NW, eps=0.0) == moe.MOE_ERR_INVALID_ARG
    assert call(nw=NW, eps=float("nan")) == moe.MOE_ERR_INVALID_ARG
    assert call(ids=A + 2) == moe.MOE_ERR_MISALIGNED
    assert call(out=A + 4096, ws=A + 0x50000000, wsb=WS_BIG) == moe.MOE_ERR_INVALID_ARG  # x
    assert call(nw=A + 0x2000000 + 64, ws=A + 0x60000000, wsb=WS_BIG) == \
        moe.MOE_ERR_INVALID_ARG                                   # norm weights inside out
    assert call(S=moe.shape(n_experts=384, top_k=8, n_shared=0), wsb=WS_BIG) == \
        moe.MOE_ERR_UNSUPPORTED
    assert call(S=moe.shape(moe.MOE_W_MXFP8), wsb=WS_BIG) == moe.MOE_ERR_UNSUPPORTED


def test_workspace_status_argument_errors():
    L = moe.lib()
    WS = A + 0x3000000
    assert L.moe_workspace_status(None, WS_BIG, A, 0) == moe.MOE_ERR_WORKSPACE
    assert L.moe_workspace_status(WS, 64, A, 0) == moe.MOE_ERR_WORKSPACE
    assert L.moe_workspace_status(WS + 16, WS_BIG, A, 0) == moe.MOE_ERR_MISALIGNED
    assert L.moe_workspace_status(WS, WS_BIG, None, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_status(WS, WS_BIG, A + 2, 0) == moe.MOE_ERR_MISALIGNED
    assert L.moe_workspace_status(WS, WS_BIG, WS + 64, 0) == moe.MOE_ERR_INVALID_ARG


def test_prefill_workspace_keeps_the_decode_region():
    """A prefill workspace is larger than the decode one by more than the
    decode region: its data starts past the region the decode kernels keep
    their counters in, so one workspace serves both (the GPU test
    test_one_workspace_serves_prefill_and_decode checks the results)."""
    d = moe.moe_workspace_bytes(8)
    for T in (1, 64, 8192):
        assert moe.moe_workspace_bytes(T, prefill=True) > d


def test_general_workspace_layout():
    S = moe.shape(moe.MOE_W_NVFP4_A4)                    # Flint's shape, W4A4: general path
    off = moe.general_workspace_layout(S)
    need = moe.moe_workspace_bytes(8, S=S)
    assert off["n_entries"] >= moe.moe_workspace_bytes(8)   # after the Flint paths' region
    assert sorted(off.values()) == [off[k] for k in ["n_entries", "entry", "amask", "h", "xq",
                                                      "gx", "hq", "gh"]]
    assert off["gh"] + 4 * 66 * 8 <= need
    with pytest.raises(moe.MoeError):
        moe.general_workspace_layout(moe.shape())        # Flint NVFP4: the fused path
    # W4A4 needs the NVFP4 scales and global (no launch: workspace too small)
    assert _forward(S=S, ws_bytes=1024) == moe.MOE_ERR_WORKSPACE
    bf = _FakeExperts(A + 0x4000000, fmt="bf16")
    assert _forward(S=S, routed=bf) == moe.MOE_ERR_INVALID_ARG
    assert _forward(S=S, prefill=True) == moe.MOE_ERR_UNSUPPORTED


def test_decode_batch_limit_is_unsupported_not_invalid():
    assert _forward(B=9) == moe.MOE_ERR_UNSUPPORTED
    assert _forward(B=64) == moe.MOE_ERR_UNSUPPORTED


def test_route_argument_errors():
    L = moe.lib()
    S = moe.shape()
    call = lambda **k: L.moe_decode_route(  # noqa: E731
        ctypes.byref(k.get("S", S)), k.get("x", A), k.get("B", 1), k.get("r", A + 0x1000000),
        k.get("ids", A + 0x2000000), k.get("w", A + 0x2100000), k.get("ws", A + 0x3000000),
        k.get("wsb", WS_BIG), 0)
    assert call(B=0) == moe.MOE_ERR_INVALID_ARG
    assert call(B=9) == moe.MOE_ERR_UNSUPPORTED
    assert call(ids=None) == moe.MOE_ERR_INVALID_ARG
    assert call(w=A + 0x2100001) == moe.MOE_ERR_MISALIGNED
    assert call(wsb=64) == moe.MOE_ERR_WORKSPACE
    assert call(x=A + 4) == moe.MOE_ERR_MISALIGNED


def test_dequant_argument_errors():
    L = moe.lib()
    X = moe.experts_struct(_FakeExperts(A))
    S = moe.shape()
    assert L.moe_nvfp4_dequant(ctypes.byref(S), ctypes.byref(X), 0, 3, A + 0x1000000, 0) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_nvfp4_dequant(ctypes.byref(S), ctypes.byref(X), -1, 0, A + 0x1000000, 0) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_nvfp4_dequant(ctypes.byref(S), ctypes.byref(X), 0, 0, None, 0) == \
        moe.MOE_ERR_INVALID_ARG
    Sb = moe.shape(moe.MOE_W_BF16)
    assert L.moe_nvfp4_dequant(ctypes.byref(Sb), ctypes.byref(X), 0, 0, A + 0x1000000, 0) == \
        moe.MOE_ERR_UNSUPPORTED


def test_convert_check_argument_errors():
    L = moe.lib()
    assert L.moe_a4_convert_check(None, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_a4_convert_check(A + 4, 0) == moe.MOE_ERR_MISALIGNED
