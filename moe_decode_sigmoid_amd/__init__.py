"""Python binding of the gfx950 MoE layer library (libmoe_decode.so).

Thin ctypes marshalling over the C ABI declared in include/moe_decode.h:
the same entry-point names, torch tensors in, device pointers and the
current HIP stream out.  Every step of the layer runs in the library's HIP
kernels; this module computes nothing.  If the library is not built, or the
GPU is missing, calls fail loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import pathlib

HERE = pathlib.Path(__file__).resolve().parent
LIB_PATH = HERE / "libmoe_decode.so"

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED = 0, -1, -2
MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = -3, -4, -5
MOE_W_NVFP4, MOE_W_BF16, MOE_W_MXFP8, MOE_W_NVFP4_A4 = 0, 1, 2, 3
HIDDEN, INTER, N_EXPERTS, TOP_K, N_SHARED = 2048, 512, 256, 6, 1
MAX_DECODE_BATCH = 8

_LIB = None


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("wfmt", ctypes.c_int32)]


class Fuse(ctypes.Structure):
    _fields_ = [("norm_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("residual", ctypes.c_void_p), ("xn_out", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("global_", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it was not built)."""
    global _LIB
    if _LIB is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(str(LIB_PATH))
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.moe_abi_version.restype = i32
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [P(Shape), i32, i32]
        L.moe_decode_route.restype = ctypes.c_int
        L.moe_decode_route.argtypes = [P(Shape), vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_decode_forward.restype = ctypes.c_int
        L.moe_decode_forward.argtypes = [P(Shape), vp, i32, vp, P(Experts), P(Experts), vp, vp,
                                         vp, vp, sz, vp]
        L.moe_decode_forward_noalloc.restype = ctypes.c_int
        L.moe_decode_forward_noalloc.argtypes = [P(Shape), vp, i32, vp, P(Experts), P(Experts),
                                                 vp, vp, vp, vp]
        L.moe_nvfp4_gemv.restype = ctypes.c_int
        L.moe_nvfp4_gemv.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.moe_decode_forward_timed.restype = ctypes.c_int
        L.moe_decode_forward_timed.argtypes = [P(Shape), vp, i32, vp, P(Experts), P(Experts), vp,
                                               vp, vp, vp, sz, vp, vp, vp]
        L.moe_prefill_forward.restype = ctypes.c_int
        L.moe_prefill_forward.argtypes = [P(Shape), vp, i32, vp, P(Experts), P(Experts), vp, vp,
                                          vp, vp, sz, vp]
        L.moe_decode_forward_ex.restype = ctypes.c_int
        L.moe_decode_forward_ex.argtypes = [P(Shape), vp, i32, P(Fuse), vp, P(Experts),
                                            P(Experts), vp, vp, vp, vp, sz, vp]
        L.moe_prefill_forward_ex.restype = ctypes.c_int
        L.moe_prefill_forward_ex.argtypes = [P(Shape), vp, i32, P(Fuse), vp, P(Experts),
                                             P(Experts), vp, vp, vp, vp, sz, vp]
        L.moe_decode_stack_forward.restype = ctypes.c_int
        L.moe_decode_stack_forward.argtypes = [P(Shape), i32, vp, vp, i32, vp, vp, vp, sz, vp]
        L.moe_decode_chain_forward.restype = ctypes.c_int
        L.moe_decode_chain_forward.argtypes = [P(Shape), i32, vp, vp, i32, vp, ctypes.c_float, vp,
                                               vp, vp, sz, vp]
        L.moe_workspace_status.restype = ctypes.c_int
        L.moe_workspace_status.argtypes = [vp, sz, vp, vp]
        L.moe_general_workspace_layout.restype = ctypes.c_int
        L.moe_general_workspace_layout.argtypes = [P(Shape), P(sz)]
        L.moe_nvfp4_dequant.restype = ctypes.c_int
        L.moe_nvfp4_dequant.argtypes = [P(Shape), P(Experts), i32, i32, vp, vp]
        L.moe_a4_convert_check.restype = ctypes.c_int
        L.moe_a4_convert_check.argtypes = [vp, vp]
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def shape(fmt: int = MOE_W_NVFP4, hidden=HIDDEN, inter=INTER, n_experts=N_EXPERTS, top_k=TOP_K,
          n_shared=N_SHARED) -> Shape:
    return Shape(hidden, inter, n_experts, top_k, n_shared, fmt)


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return {"nvfp4": MOE_W_NVFP4, "bf16": MOE_W_BF16, "mxfp8": MOE_W_MXFP8,
                "nvfp4_a4": MOE_W_NVFP4_A4}[fmt]
    return int(fmt)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ref(st):
    return None if st is None else ctypes.byref(st)


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def experts_struct(ex) -> Experts | None:
    """ex: object with w13, w2 and (NVFP4) w13_scale, w2_scale, glob device
    tensors, (MXFP8) w13_scale, w2_scale; None (no shared expert) -> None."""
    if ex is None:
        return None
    return Experts(_ptr(ex.w13), _ptr(getattr(ex, "w13_scale", None)), _ptr(ex.w2),
                   _ptr(getattr(ex, "w2_scale", None)), _ptr(getattr(ex, "glob", None)))


def abi_version() -> int:
    return int(lib().moe_abi_version())


def moe_workspace_bytes(tokens: int, prefill: bool = False, fmt=MOE_W_NVFP4,
                        S: Shape | None = None) -> int:
    S = S or shape(_fmt(fmt))
    return int(lib().moe_workspace_bytes(ctypes.byref(S), tokens, 1 if prefill else 0))


def moe_decode_route(x, router_w, ids, w, ws, fmt=MOE_W_NVFP4, stream=None, S: Shape | None = None):
    """Router + top-k for x bf16 [B, H]; writes ids int32 [B, k] and w f32 [B, k]."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if hasattr(x, "shape") else 1
    st = lib().moe_decode_route(ctypes.byref(S), _ptr(x), B, _ptr(router_w), _ptr(ids), _ptr(w),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_decode_route")


def moe_decode_forward(x, router_w, routed, shared, out, ws, ids_out=None, w_out=None,
                       fmt=MOE_W_NVFP4, stream=None, S: Shape | None = None, B: int | None = None):
    """The layer for x bf16 [B, H] (B <= 8) into out bf16 [B, H]."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if B is None else B
    R, Sh = experts_struct(routed), experts_struct(shared)
    st = lib().moe_decode_forward(ctypes.byref(S), _ptr(x), B, _ptr(router_w), ctypes.byref(R),
                                  _ref(Sh), _ptr(out), _ptr(ids_out), _ptr(w_out),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_decode_forward")


def moe_decode_forward_noalloc(x, router_w, routed, shared, out, ids_out=None, w_out=None,
                               fmt=MOE_W_NVFP4, stream=None, S: Shape | None = None,
                               B: int | None = None):
    """moe_decode_forward on the library's own per-GPU workspace (no workspace
    argument, no allocation); calls on one GPU must not overlap."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if B is None else B
    R, Sh = experts_struct(routed), experts_struct(shared)
    st = lib().moe_decode_forward_noalloc(ctypes.byref(S), _ptr(x), B, _ptr(router_w),
                                          ctypes.byref(R), _ref(Sh), _ptr(out), _ptr(ids_out),
                                          _ptr(w_out), _stream(stream))
    _check(st, "moe_decode_forward_noalloc")


def moe_decode_forward_timed(x, router_w, routed, shared, out, ws, ev_start, ev_stop,
                             ids_out=None, w_out=None, fmt=MOE_W_NVFP4, stream=None,
                             S: Shape | None = None, B: int | None = None):
    """moe_decode_forward recording the kernel's own start / end on two
    torch.cuda.Event(enable_timing=True) (ev_start.elapsed_time(ev_stop) after
    a synchronize is the kernel's execution time)."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if B is None else B
    R, Sh = experts_struct(routed), experts_struct(shared)
    import torch
    for ev in (ev_start, ev_stop):
        if not ev.cuda_event:           # torch creates its events at their first record
            ev.record(torch.cuda.current_stream())
    st = lib().moe_decode_forward_timed(ctypes.byref(S), _ptr(x), B, _ptr(router_w),
                                        ctypes.byref(R), _ref(Sh), _ptr(out),
                                        _ptr(ids_out), _ptr(w_out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream),
                                        ctypes.c_void_p(ev_start.cuda_event),
                                        ctypes.c_void_p(ev_stop.cuda_event))
    _check(st, "moe_decode_forward_timed")


def moe_nvfp4_gemv(x, codes, scales, glob, y, stream=None, B: int | None = None):
    """Dense NVFP4 GEMV: x bf16 [B, K], codes u8 [N, K/2], scales u8 [N, K/16],
    glob f32 [1] (device) -> y bf16 [B, N]."""
    B = x.shape[0] if B is None else B
    K = x.shape[-1]
    N = codes.shape[0]
    st = lib().moe_nvfp4_gemv(_ptr(x), B, K, N, _ptr(codes), _ptr(scales), _ptr(glob), _ptr(y),
                              _stream(stream))
    _check(st, "moe_nvfp4_gemv")


def moe_prefill_forward(x, router_w, routed, shared, out, ws, ids_out=None, w_out=None,
                        fmt=MOE_W_NVFP4, stream=None, S: Shape | None = None, T: int | None = None):
    """The layer for x bf16 [T, H] at prefill sizes into out bf16 [T, H]."""
    S = S or shape(_fmt(fmt))
    T = x.shape[0] if T is None else T
    R, Sh = experts_struct(routed), experts_struct(shared)
    st = lib().moe_prefill_forward(ctypes.byref(S), _ptr(x), T, _ptr(router_w), ctypes.byref(R),
                                   _ref(Sh), _ptr(out), _ptr(ids_out), _ptr(w_out),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_prefill_forward")


def fuse_struct(norm_w=None, eps: float = 1e-6, residual=None, xn_out=None) -> Fuse:
    """The fused neighbours: RMSNorm weight bf16 [H] and epsilon, residual
    bf16 [T, H], normalised-input output bf16 [T, H] (each None = off)."""
    return Fuse(_ptr(norm_w), float(eps), _ptr(residual), _ptr(xn_out))


def moe_decode_forward_ex(x, router_w, routed, shared, out, ws, norm_w=None, eps: float = 1e-6,
                          residual=None, xn_out=None, ids_out=None, w_out=None, fmt=MOE_W_NVFP4,
                          stream=None, S: Shape | None = None, B: int | None = None):
    """out = residual + layer(rmsnorm(x)) for x bf16 [B, H] (B <= 8), each part optional."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if B is None else B
    R, Sh = experts_struct(routed), experts_struct(shared)
    F = fuse_struct(norm_w, eps, residual, xn_out)
    st = lib().moe_decode_forward_ex(ctypes.byref(S), _ptr(x), B, ctypes.byref(F),
                                     _ptr(router_w), ctypes.byref(R), _ref(Sh),
                                     _ptr(out), _ptr(ids_out), _ptr(w_out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_decode_forward_ex")


def moe_prefill_forward_ex(x, router_w, routed, shared, out, ws, norm_w=None, eps: float = 1e-6,
                           residual=None, xn_out=None, ids_out=None, w_out=None,
                           fmt=MOE_W_NVFP4, stream=None, S: Shape | None = None,
                           T: int | None = None):
    """out = residual + layer(rmsnorm(x)) for x bf16 [T, H] at prefill sizes."""
    S = S or shape(_fmt(fmt))
    T = x.shape[0] if T is None else T
    R, Sh = experts_struct(routed), experts_struct(shared)
    F = fuse_struct(norm_w, eps, residual, xn_out)
    st = lib().moe_prefill_forward_ex(ctypes.byref(S), _ptr(x), T, ctypes.byref(F),
                                      _ptr(router_w), ctypes.byref(R), _ref(Sh),
                                      _ptr(out), _ptr(ids_out), _ptr(w_out), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_prefill_forward_ex")


def general_workspace_layout(S: Shape) -> dict:
    """Byte offsets of the general decode path's workspace regions (diagnostics)."""
    off = (ctypes.c_size_t * 8)()
    _check(lib().moe_general_workspace_layout(ctypes.byref(S), off), "moe_general_workspace_layout")
    keys = ["n_entries", "entry", "amask", "h", "xq", "gx", "hq", "gh"]
    return {k: int(v) for k, v in zip(keys, off)}


def layer_table(device_layers, device="cuda"):
    """A device array of moe_layer records (int64 [L, 11]: router, then the
    routed and shared sets' w13, w13_scale, w2, w2_scale, global) for
    moe_decode_stack_forward; the tensors it points to must stay alive."""
    import torch
    rows = []
    for d in device_layers:
        r = experts_struct(d.routed)
        sh = experts_struct(d.shared)
        rows.append([_ptr(d.router) or 0] +
                    [v or 0 for v in (r.w13, r.w13_scale, r.w2, r.w2_scale, r.global_)] +
                    [v or 0 for v in (sh.w13, sh.w13_scale, sh.w2, sh.w2_scale, sh.global_)])
    return torch.tensor(rows, dtype=torch.int64).to(device)


def moe_decode_stack_forward(x, table, out, ws, ids_out=None, fmt=MOE_W_NVFP4, stream=None,
                             S: Shape | None = None, B: int | None = None):
    """n_layers = table.shape[0] independent layers on the same x bf16 [B, H],
    one launch: out bf16 [L, B, H] (ids_out int32 [L, B, k] optional)."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if B is None else B
    st = lib().moe_decode_stack_forward(ctypes.byref(S), table.shape[0], _ptr(table), _ptr(x), B,
                                        _ptr(out), _ptr(ids_out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_decode_stack_forward")


def moe_decode_chain_forward(x, table, out, ws, norm_w=None, eps: float = 1e-6, ids_out=None,
                             fmt=MOE_W_NVFP4, stream=None, S: Shape | None = None,
                             B: int | None = None):
    """A chained residual stack of n_layers = table.shape[0] layers in one launch:
    x_0 = x bf16 [B, H], x_{l+1} = x_l + layer_l(rmsnorm_l(x_l)) into out bf16
    [L, B, H] (norm_w bf16 [L, H] or None; ids_out int32 [L, B, k] optional)."""
    S = S or shape(_fmt(fmt))
    B = x.shape[0] if B is None else B
    st = lib().moe_decode_chain_forward(ctypes.byref(S), table.shape[0], _ptr(table), _ptr(x), B,
                                        _ptr(norm_w), float(eps), _ptr(out), _ptr(ids_out),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_decode_chain_forward")


def moe_workspace_status(ws, status, stream=None):
    """Enqueue the copy of the workspace's wait-status word into status (device
    int32 [1]) and clear the word; nonzero after a synchronize means a bounded
    wait of a single-launch decode call gave up and its output is invalid."""
    st = lib().moe_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), _ptr(status),
                                    _stream(stream))
    _check(st, "moe_workspace_status")


def moe_a4_convert_check(counts, stream=None):
    """The W4A4 quantiser's hardware roundings against their definitions over
    every fp32 bit pattern; counts: int64 [2] on the device, overwritten with
    the E2M1 and E4M3 mismatch counts."""
    st = lib().moe_a4_convert_check(_ptr(counts), _stream(stream))
    _check(st, "moe_a4_convert_check")


def moe_nvfp4_dequant(expert_set, expert: int, tensor: int, out, stream=None):
    """Decode tensor (0 gate, 1 up, 2 down) of one expert of an NVFP4 set into out f32."""
    S = shape(MOE_W_NVFP4)
    X = experts_struct(expert_set)
    st = lib().moe_nvfp4_dequant(ctypes.byref(S), ctypes.byref(X), expert, tensor, _ptr(out),
                                 _stream(stream))
    _check(st, "moe_nvfp4_dequant")


from .device import DeviceExperts, DeviceLayer, alloc_workspace  # noqa: E402,F401
