"""fp64 CPU oracle of the Flint-style MoE decode layer (ctypes front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
The arithmetic lives in ``moe_oracle.c`` (plain C, fp64); its header lists the
passages of the Flint pages each step follows.  Inputs are numpy arrays in the
layouts the input generator writes (bf16 as ``np.uint16`` bit patterns).
"""
from __future__ import annotations

import ctypes
import pathlib

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
_LIB = None


class _Experts(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13s", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2s", ctypes.c_void_p), ("glob", ctypes.c_void_p), ("fmt", ctypes.c_int32)]


class _Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32)]


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = HERE / "libmoe_oracle.so"
        if not path.exists():
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(str(path))
        d, vp, i32, i64, f32 = (ctypes.c_double, ctypes.c_void_p, ctypes.c_int32,
                                ctypes.c_int64, ctypes.c_float)
        L.or_e2m1.restype = d
        L.or_e2m1.argtypes = [ctypes.c_uint8]
        L.or_e4m3.restype = d
        L.or_e4m3.argtypes = [ctypes.c_uint8]
        L.or_e8m0.restype = d
        L.or_e8m0.argtypes = [ctypes.c_uint8]
        L.or_bf16.restype = d
        L.or_bf16.argtypes = [ctypes.c_uint16]
        L.or_sigmoid.restype = d
        L.or_sigmoid.argtypes = [d]
        L.or_dequant_f32.argtypes = [vp, vp, f32, i64, i64, vp]
        L.or_dequant_f64.argtypes = [vp, vp, f32, i64, i64, vp]
        L.or_router_logits.argtypes = [vp, vp, i32, i32, vp]
        L.or_topk.argtypes = [vp, i32, i32, vp, vp]
        L.or_route.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, vp, vp, vp, vp]
        L.or_expert.argtypes = [ctypes.POINTER(_Shape), ctypes.POINTER(_Experts), i32, vp, vp]
        L.or_forward.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, ctypes.POINTER(_Experts),
                                 ctypes.POINTER(_Experts), vp, vp, vp, vp, vp]
        L.or_forward_dense.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp,
                                       ctypes.POINTER(_Experts), ctypes.POINTER(_Experts), vp]
        L.or_gemv_nvfp4.argtypes = [vp, i32, i32, i32, vp, vp, f32, vp]
        L.or_bf16_rne.restype = ctypes.c_uint16
        L.or_bf16_rne.argtypes = [d]
        L.or_bf16_rne_array.argtypes = [vp, i64, vp]
        L.or_rmsnorm_bf16.argtypes = [vp, i32, i32, vp, d, vp]
        L.or_quant_fp4_46.argtypes = [vp, i64, vp, vp, vp, vp]
        L.or_forward_w4a4.argtypes = [ctypes.POINTER(_Shape), vp, i32, vp, ctypes.POINTER(_Experts),
                                      ctypes.POINTER(_Experts), vp, vp, vp, vp, vp, vp, vp]
        L.or_num_threads.restype = ctypes.c_int
        L.or_set_num_threads.argtypes = [ctypes.c_int]
        _LIB = L
    return _LIB


def _p(a) -> int:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _experts(X) -> _Experts:
    """X: an object with fmt ('nvfp4' | 'bf16' | 'mxfp8'), w13, w2 and, for
    nvfp4, w13_scale, w2_scale, glob; for mxfp8, w13_scale, w2_scale (the
    input generator's Experts)."""
    if X.fmt == "nvfp4":
        return _Experts(_p(X.w13), _p(X.w13_scale), _p(X.w2), _p(X.w2_scale), _p(X.glob), 0)
    if X.fmt == "mxfp8":
        return _Experts(_p(X.w13), _p(X.w13_scale), _p(X.w2), _p(X.w2_scale), None, 2)
    return _Experts(_p(X.w13), None, _p(X.w2), None, None, 1)


def _shape(H, I, E, K, n_shared=1) -> _Shape:
    return _Shape(H, I, E, K, n_shared)


# ----------------------------------------------------------------- formats
def e2m1(nibble: int) -> float:
    return float(lib().or_e2m1(nibble))


def e4m3(byte: int) -> float:
    return float(lib().or_e4m3(byte))


def e8m0(byte: int) -> float:
    return float(lib().or_e8m0(byte))


def bf16(bits: int) -> float:
    return float(lib().or_bf16(bits))


def sigmoid(z: float) -> float:
    return float(lib().or_sigmoid(z))


def dequant_f32(codes: np.ndarray, scales: np.ndarray, glob: float) -> np.ndarray:
    """fp32(e2m1 * e4m3 * global) for a [rows, cols/2] code tensor."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, half * 2), np.float32)
    lib().or_dequant_f32(_p(codes), _p(scales), glob, rows, half * 2, _p(out))
    return out


def dequant_f64(codes: np.ndarray, scales: np.ndarray, glob: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, half * 2), np.float64)
    lib().or_dequant_f64(_p(codes), _p(scales), glob, rows, half * 2, _p(out))
    return out


# ----------------------------------------------------------------- routing
def router_logits(x: np.ndarray, router: np.ndarray) -> np.ndarray:
    """x u16 [H]; router u16 [E, H] -> fp64 [E]."""
    x = np.ascontiguousarray(x, np.uint16)
    router = np.ascontiguousarray(router, np.uint16)
    E, H = router.shape
    out = np.empty(E, np.float64)
    lib().or_router_logits(_p(x), _p(router), E, H, _p(out))
    return out


def topk(scores: np.ndarray, k: int):
    scores = np.ascontiguousarray(scores, np.float64)
    ids = np.empty(k, np.int32)
    gap = np.zeros(1, np.float64)
    lib().or_topk(_p(scores), scores.size, k, _p(ids), _p(gap))
    return ids, float(gap[0])


def route(x: np.ndarray, router: np.ndarray, k: int):
    """x u16 [B, H] -> ids i32 [B, k], w f64 [B, k], gap f64 [B], scores f64 [B, E]."""
    x = np.ascontiguousarray(x, np.uint16)
    router = np.ascontiguousarray(router, np.uint16)
    B, H = x.shape
    E = router.shape[0]
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    gap = np.empty(B, np.float64)
    scores = np.empty((B, E), np.float64)
    S = _shape(H, 0, E, k)
    lib().or_route(ctypes.byref(S), _p(x), B, _p(router), _p(ids), _p(w), _p(gap), _p(scores))
    return ids, w, gap, scores


# ----------------------------------------------------------------- layer
def expert(X, e: int, x: np.ndarray, H: int, I: int) -> np.ndarray:
    """D_e(SiLU(G_e x) * U_e x) for one fp64 token x [H]."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(H, np.float64)
    S = _shape(H, I, X.n, 1)
    XE = _experts(X)
    lib().or_expert(ctypes.byref(S), ctypes.byref(XE), e, _p(x), _p(out))
    return out


def forward(x: np.ndarray, router: np.ndarray, routed, shared, k: int, I: int,
            forced_ids: np.ndarray | None = None):
    """The layer for x u16 [B, H].  Returns (y f64 [B, H], ids [B, k], w [B, k], gap [B])."""
    x = np.ascontiguousarray(x, np.uint16)
    router = np.ascontiguousarray(router, np.uint16)
    B, H = x.shape
    E = router.shape[0]
    y = np.empty((B, H), np.float64)
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    gap = np.empty(B, np.float64)
    forced = None
    if forced_ids is not None:
        forced = np.ascontiguousarray(forced_ids, np.int32)
        assert forced.shape == (B, k)
    S = _shape(H, I, E, k, shared.n if shared is not None else 0)
    R = _experts(routed)
    Sh = _experts(shared) if shared is not None else _experts(routed)
    lib().or_forward(ctypes.byref(S), _p(x), B, _p(router), ctypes.byref(R), ctypes.byref(Sh),
                     _p(forced), _p(y), _p(ids), _p(w), _p(gap))
    return y, ids, w, gap


def forward_dense(x: np.ndarray, router: np.ndarray, routed, shared, k: int, I: int) -> np.ndarray:
    x = np.ascontiguousarray(x, np.uint16)
    router = np.ascontiguousarray(router, np.uint16)
    B, H = x.shape
    E = router.shape[0]
    y = np.empty((B, H), np.float64)
    S = _shape(H, I, E, k, shared.n if shared is not None else 0)
    R = _experts(routed)
    Sh = _experts(shared) if shared is not None else _experts(routed)
    lib().or_forward_dense(ctypes.byref(S), _p(x), B, _p(router), ctypes.byref(R),
                           ctypes.byref(Sh), _p(y))
    return y


def forward_layer(x: np.ndarray, layer, forced_ids=None):
    """Convenience: the layer for an input generator Layer object."""
    return forward(x, layer.router, layer.routed, layer.shared, layer.K, layer.I, forced_ids)


# ----------------------------------------------------------------- dense GEMV
def gemv_nvfp4(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, glob: float) -> np.ndarray:
    """x u16 [B, K]; codes u8 [N, K/2]; scales u8 [N, K/16] -> fp64 [B, N] = x . W^T."""
    x = np.ascontiguousarray(x, np.uint16)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    B, K = x.shape
    N = codes.shape[0]
    assert codes.shape == (N, K // 2) and scales.shape == (N, K // 16)
    out = np.empty((B, N), np.float64)
    lib().or_gemv_nvfp4(_p(x), B, K, N, _p(codes), _p(scales), glob, _p(out))
    return out


# ----------------------------------------------------------------- RMSNorm + residual
def bf16_rne(v) -> np.ndarray:
    """fp64 values rounded once to bf16 (ties to even) -> u16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(v, np.float64))
    out = np.empty(a.shape, np.uint16)
    lib().or_bf16_rne_array(_p(a), a.size, _p(out))
    return out


def rmsnorm_bf16(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x u16 [T, H], w u16 [H] -> u16 [T, H]: x * w / sqrt(mean x^2 + eps), rounded to bf16."""
    x = np.ascontiguousarray(x, np.uint16)
    w = np.ascontiguousarray(w, np.uint16)
    T, H = x.shape
    assert w.shape == (H,)
    out = np.empty((T, H), np.uint16)
    lib().or_rmsnorm_bf16(_p(x), T, H, _p(w), float(eps), _p(out))
    return out


def forward_fused(x: np.ndarray, layer, norm_w=None, eps: float = 0.0, residual=None,
                  xn=None, forced_ids=None):
    """The layer with its neighbours fused: out = residual + layer(rmsnorm(x)).
    norm_w None skips the norm; residual None adds nothing.  xn, when given,
    replaces the oracle's own normalised input (u16 [B, H]), so that routing
    decisions can be taken on the same bf16 input as another implementation.
    Returns (out f64 [B, H], ids, w, gap, the normalised input u16 [B, H])."""
    x = np.ascontiguousarray(x, np.uint16)
    if xn is None:
        xn = rmsnorm_bf16(x, norm_w, eps) if norm_w is not None else x
    y, ids, w, gap = forward_layer(xn, layer, forced_ids)
    if residual is not None:
        r = np.ascontiguousarray(residual, np.uint16).astype(np.uint32) << 16
        y = y + r.view(np.float32).astype(np.float64)
    return y, ids, w, gap, xn


# ----------------------------------------------------------------- W4A4 (Four Over Six)
def quant_fp4_46(v) -> tuple:
    """One vector (float32, length a multiple of 16) -> (codes u8 [n], scales
    u8 [n/16], global float, exact values f64 [n])."""
    v = np.ascontiguousarray(np.asarray(v, np.float32))
    n = v.size
    codes = np.empty(n, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    g = np.zeros(1, np.float32)
    out = np.empty(n, np.float64)
    lib().or_quant_fp4_46(_p(v), n, _p(codes), _p(scales), _p(g), _p(out))
    return codes, scales, float(g[0]), out


def forward_w4a4(x: np.ndarray, layer, forced_ids=None, h_in=None):
    """The W4A4 layer (NVFP4 weights, Four-Over-Six NVFP4 activations) for x
    u16 [B, H].  h_in: u16 [B, k + n_shared, I] (routed ids ascending, then
    shared) replacing the oracle's bf16 h before its quantisation.
    Returns (y f64 [B, H], ids, w, gap, h u16 [B, k + n_shared, I])."""
    x = np.ascontiguousarray(x, np.uint16)
    B, H = x.shape
    k, I = layer.K, layer.I
    ns = layer.shared.n if layer.shared is not None else 0
    y = np.empty((B, H), np.float64)
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    gap = np.empty(B, np.float64)
    h_out = np.empty((B, k + ns, I), np.uint16)
    forced = None if forced_ids is None else np.ascontiguousarray(forced_ids, np.int32)
    hin = None if h_in is None else np.ascontiguousarray(h_in, np.uint16)
    S = _shape(H, I, layer.router.shape[0], k, ns)
    R = _experts(layer.routed)
    Sh = _experts(layer.shared) if layer.shared is not None else _experts(layer.routed)
    lib().or_forward_w4a4(ctypes.byref(S), _p(x), B, _p(layer.router), ctypes.byref(R),
                          ctypes.byref(Sh), _p(forced), _p(hin), _p(y), _p(ids), _p(w), _p(gap),
                          _p(h_out))
    return y, ids, w, gap, h_out


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    lib().or_set_num_threads(n)
