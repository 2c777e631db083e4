"""Seeded synthetic inputs for the MoE decode layer (numpy front end).

The heavy lifting (splitmix64 streams, Irwin-Hall normals, bf16 rounding and
NVFP4 packing) lives in ``testgen.c``; see its header for the exact recipe.
This module holds none of the layer's arithmetic: it produces inputs that the
fp64 oracle and the HIP library both consume.

Arrays are numpy, host side.  bf16 tensors are ``np.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import dataclasses
import pathlib

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
_LIB = None

# Tensor ids of the random streams.
T_ROUTER, T_GATE, T_UP, T_DOWN, T_X, T_DENSE = 0, 1, 2, 3, 4, 5

HIDDEN, INTER, N_EXPERTS, TOP_K = 2048, 512, 256, 6
SIGMA_W = 0.02


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = HERE / "libtestgen.so"
        if not path.exists():
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(str(path))
        u64, i32, i64, f32, vp = (ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_void_p)
        L.tg_splitmix_at.restype = u64
        L.tg_splitmix_at.argtypes = [u64, u64]
        L.tg_stream_key.restype = u64
        L.tg_stream_key.argtypes = [u64, i32, i32, i32]
        L.tg_bf16_rne.restype = ctypes.c_uint16
        L.tg_bf16_rne.argtypes = [f32]
        L.tg_normal_bf16.argtypes = [u64, i32, i32, i32, f32, i64, vp]
        L.tg_normal_f32.argtypes = [u64, i32, i32, i32, i64, vp]
        L.tg_e4m3_encode.restype = ctypes.c_uint8
        L.tg_e4m3_encode.argtypes = [f32, ctypes.POINTER(f32)]
        L.tg_e2m1_encode.restype = ctypes.c_uint8
        L.tg_e2m1_encode.argtypes = [f32]
        L.tg_quantize_nvfp4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.tg_make_experts_nvfp4.argtypes = [u64, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp]
        L.tg_make_experts_bf16.argtypes = [u64, i32, i32, i32, i32, i32, f32, vp, vp]
        L.tg_quantize_mxfp8.argtypes = [vp, i64, i64, vp, vp]
        L.tg_make_experts_mxfp8.argtypes = [u64, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp]
        L.tg_make_router.argtypes = [u64, i32, i32, i32, f32, vp]
        L.tg_make_x.argtypes = [u64, i32, i32, vp]
        L.tg_num_threads.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ----------------------------------------------------------------- scalars
def splitmix_at(key: int, n: int) -> int:
    return int(lib().tg_splitmix_at(key, n))


def stream_key(seed: int, layer: int, expert: int, tensor: int) -> int:
    return int(lib().tg_stream_key(seed, layer, expert, tensor))


def bf16_rne(f: float) -> int:
    return int(lib().tg_bf16_rne(f))


def e4m3_encode(s: float) -> tuple[int, float]:
    q = ctypes.c_float(0.0)
    b = lib().tg_e4m3_encode(s, ctypes.byref(q))
    return int(b), float(q.value)


def e2m1_encode(v: float) -> int:
    return int(lib().tg_e2m1_encode(v))


# ----------------------------------------------------------------- tensors
def normal_bf16(seed: int, layer: int, expert: int, tensor: int, sigma: float, n: int) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().tg_normal_bf16(seed, layer, expert, tensor, sigma, n, _p(out))
    return out


def normal_f32(seed: int, layer: int, expert: int, tensor: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().tg_normal_f32(seed, layer, expert, tensor, n, _p(out))
    return out


def quantize_nvfp4(w_bf16: np.ndarray):
    """Pack a bf16 [rows, cols] tensor: (codes u8 [rows, cols/2], scales u8 [rows, cols/16], global f32)."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    rows, cols = w.shape
    assert cols % 16 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    g = np.zeros(1, np.float32)
    lib().tg_quantize_nvfp4(_p(w), rows, cols, _p(codes), _p(scales), _p(g))
    return codes, scales, float(g[0])


def make_x(seed: int, T: int, H: int = HIDDEN) -> np.ndarray:
    out = np.empty((T, H), np.uint16)
    lib().tg_make_x(seed, T, H, _p(out))
    return out


def make_router(seed: int, layer: int, E: int = N_EXPERTS, H: int = HIDDEN,
                sigma: float = SIGMA_W) -> np.ndarray:
    out = np.empty((E, H), np.uint16)
    lib().tg_make_router(seed, layer, E, H, sigma, _p(out))
    return out


def make_dense(seed: int, layer: int, which: int, N: int, K: int, sigma: float = SIGMA_W):
    """A dense [N, K] weight ~ N(0, sigma) (bf16), packed to NVFP4: (codes u8 [N, K/2],
    scales u8 [N, K/16], global f32).  `which` tells apart matrices of one layer."""
    w = normal_bf16(seed, layer, which, T_DENSE, sigma, N * K).reshape(N, K)
    return quantize_nvfp4(w)


@dataclasses.dataclass
class Experts:
    """One expert set.  fmt 'nvfp4': w13 u8 [n,2,I,H/2], w13_scale u8 [n,2,I,H/16],
    w2 u8 [n,H,I/2], w2_scale u8 [n,H,I/16], glob f32 [n,3].
    fmt 'mxfp8': w13 u8 [n,2,I,H] (E4M3), w13_scale u8 [n,2,I,H/32] (E8M0),
    w2 u8 [n,H,I], w2_scale u8 [n,H,I/32] (glob None).
    fmt 'bf16': w13 u16 [n,2,I,H], w2 u16 [n,H,I] (scales and glob None)."""
    fmt: str
    n: int
    w13: np.ndarray
    w2: np.ndarray
    w13_scale: np.ndarray | None = None
    w2_scale: np.ndarray | None = None
    glob: np.ndarray | None = None


def make_experts(seed: int, layer: int, e0: int, n: int, H: int = HIDDEN, I: int = INTER,
                 fmt: str = "nvfp4", sigma: float = SIGMA_W) -> Experts:
    if fmt == "nvfp4":
        w13 = np.empty((n, 2, I, H // 2), np.uint8)
        w13s = np.empty((n, 2, I, H // 16), np.uint8)
        w2 = np.empty((n, H, I // 2), np.uint8)
        w2s = np.empty((n, H, I // 16), np.uint8)
        g = np.empty((n, 3), np.float32)
        lib().tg_make_experts_nvfp4(seed, layer, e0, n, H, I, sigma, _p(w13), _p(w13s), _p(w2),
                                    _p(w2s), _p(g))
        return Experts("nvfp4", n, w13, w2, w13s, w2s, g)
    if fmt == "mxfp8":
        w13 = np.empty((n, 2, I, H), np.uint8)
        w13s = np.empty((n, 2, I, H // 32), np.uint8)
        w2 = np.empty((n, H, I), np.uint8)
        w2s = np.empty((n, H, I // 32), np.uint8)
        lib().tg_make_experts_mxfp8(seed, layer, e0, n, H, I, sigma, _p(w13), _p(w13s), _p(w2),
                                    _p(w2s))
        return Experts("mxfp8", n, w13, w2, w13s, w2s, None)
    if fmt == "bf16":
        w13 = np.empty((n, 2, I, H), np.uint16)
        w2 = np.empty((n, H, I), np.uint16)
        lib().tg_make_experts_bf16(seed, layer, e0, n, H, I, sigma, _p(w13), _p(w2))
        return Experts("bf16", n, w13, w2)
    raise ValueError(fmt)


@dataclasses.dataclass
class Layer:
    H: int
    I: int
    E: int
    K: int
    router: np.ndarray          # u16 [E, H]
    routed: Experts             # n = E
    shared: Experts | None      # n = n_shared (stream expert ids E ..), None if none


def make_layer(seed: int, layer: int = 0, fmt: str = "nvfp4", H: int = HIDDEN, I: int = INTER,
               E: int = N_EXPERTS, K: int = TOP_K, sigma: float = SIGMA_W,
               n_shared: int = 1) -> Layer:
    """Shared experts take expert ids E .. E + n_shared - 1 of the stream key
    (none when n_shared is 0: then `shared` is None)."""
    router = make_router(seed, layer, E, H, sigma)
    routed = make_experts(seed, layer, 0, E, H, I, fmt, sigma)
    shared = make_experts(seed, layer, E, n_shared, H, I, fmt, sigma) if n_shared > 0 else None
    return Layer(H, I, E, K, router, routed, shared)


def quantize_mxfp8(w_bf16: np.ndarray):
    """Pack a bf16 [rows, cols] tensor to MXFP8: (E4M3 u8 [rows, cols], E8M0 u8 [rows, cols/32])."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    rows, cols = w.shape
    assert cols % 32 == 0
    el = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    lib().tg_quantize_mxfp8(_p(w), rows, cols, _p(el), _p(sc))
    return el, sc


def num_threads() -> int:
    return int(lib().tg_num_threads())
