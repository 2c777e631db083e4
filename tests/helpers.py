"""Test-side helpers: golden-file parsing and bf16 bit views (no layer arithmetic)."""
from __future__ import annotations

import math
import pathlib

import numpy as np

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def bf16_bits_to_f32(u16) -> np.ndarray:
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_exact(values) -> np.ndarray:
    """Bit patterns of float values that must be exactly representable in bf16."""
    f = np.asarray(values, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _num(tok: str) -> float:
    return math.nan if tok.lower() == "nan" else float(tok)


def load_table(name: str) -> dict[int, float]:
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        k, v = line.split()
        out[int(k, 0)] = _num(v)
    return out


def load_nvfp4_blocks():
    """Parse nvfp4_blocks.txt -> list of dict(rows, cols, glob, w [rows, cols] f32,
    scales u8 [rows, cols/16], codes u8 [rows, cols/2])."""
    tensors = []
    cur = None
    for line in (GOLDEN / "nvfp4_blocks.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tag, *rest = line.split()
        if tag == "tensor":
            cur = dict(rows=int(rest[0]), cols=int(rest[1]), glob=float(rest[2]), w=[])
            tensors.append(cur)
        elif tag == "w":
            cur["w"].append([float(t) for t in rest])
        elif tag == "scales":
            cur["scales"] = np.array([int(t, 16) for t in rest], np.uint8).reshape(
                cur["rows"], cur["cols"] // 16)
        elif tag == "codes":
            cur["codes"] = np.array([int(t, 16) for t in rest], np.uint8).reshape(
                cur["rows"], cur["cols"] // 2)
    for t in tensors:
        t["w"] = np.array(t["w"], np.float32).reshape(t["rows"], t["cols"])
    return tensors
