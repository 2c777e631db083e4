"""Pins of the NVFP4 pieces: oracle decode against the OCP tables, the input
generator's packer against hand-packed blocks, and round trips between them.

Cited formats: NVFP4 as the Flint pages name it ("Day-0 Support for Flint on
vLLM", Model architecture: the checkpoint runs weight-only W4A16), with
16-element blocks and FP4 maximum 6 (Inkling-2-Small article, 48-layer MoE
section); E2M1 and E4M3FN per the OCP MX v1.0 and OFP8 v1.0 specifications.
"""
import math

import numpy as np
import pytest

import oracle
import testgen
from tests.helpers import bf16_bits_to_f32, f32_to_bf16_bits_exact, load_nvfp4_blocks, load_table


def _same(a: float, b: float) -> bool:
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_decode_matches_ocp_table():
    table = load_table("e2m1_values.txt")
    assert len(table) == 16
    for code, val in table.items():
        assert _same(oracle.e2m1(code), val), (code, oracle.e2m1(code), val)


def test_e4m3_decode_matches_ocp_table():
    table = load_table("e4m3_values.txt")
    for byte, val in table.items():
        assert _same(oracle.e4m3(byte), val), (hex(byte), oracle.e4m3(byte), val)


def test_e4m3_decode_structure_exhaustive():
    vals = [oracle.e4m3(b) for b in range(256)]
    pos = vals[:127]                            # 0x00..0x7E: every non-negative finite value
    assert all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert math.isnan(vals[0x7F]) and math.isnan(vals[0xFF])
    for b in range(127):                        # sign symmetry
        assert _same(vals[b | 0x80], -vals[b])
    # subnormal step 2^-9, then 8 values per binade with step 2^(e-3)
    assert all(vals[b] == b * 2.0 ** -9 for b in range(8))
    for e in range(-6, 9):
        base = (e + 7) << 3
        for m in range(8):
            if base + m <= 0x7E:
                assert vals[base + m] == (1 + m / 8) * 2.0 ** e
    assert max(pos) == 448.0


def test_e2m1_grid_and_maximum():
    vals = sorted({abs(oracle.e2m1(c)) for c in range(16)})
    assert vals == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # FP4 maximum 6


@pytest.mark.parametrize("idx", range(4))
def test_packer_matches_hand_packed_blocks(idx):
    t = load_nvfp4_blocks()[idx]
    w = f32_to_bf16_bits_exact(t["w"])
    codes, scales, g = testgen.quantize_nvfp4(w)
    assert g == t["glob"]
    np.testing.assert_array_equal(scales, t["scales"])
    np.testing.assert_array_equal(codes, t["codes"])


@pytest.mark.parametrize("idx", range(4))
def test_oracle_dequant_of_hand_packed_blocks(idx):
    """Decoding the hand-packed bytes gives E2M1 * E4M3 * global from the spec tables."""
    t = load_nvfp4_blocks()[idx]
    e2 = load_table("e2m1_values.txt")
    rows, cols = t["rows"], t["cols"]
    expect = np.empty((rows, cols))
    e4 = {b: oracle.e4m3(b) for b in range(256)}
    for r in range(rows):
        for c in range(cols):
            byte = int(t["codes"][r, c // 2])
            nib = byte & 15 if c % 2 == 0 else byte >> 4
            expect[r, c] = e2[nib] * e4[int(t["scales"][r, c // 16])] * t["glob"]
    got = oracle.dequant_f64(t["codes"], t["scales"], t["glob"])
    np.testing.assert_array_equal(got, expect)
    if idx == 0:                       # every entry of tensor A sits on the grid
        np.testing.assert_array_equal(got, t["w"])


def test_dequant_f32_is_single_rounding_of_exact_product():
    """fp32(e2m1 * e4m3 * global) for every (nibble, scale byte) pair, with an
    awkward global so that the product needs rounding."""
    e2 = load_table("e2m1_values.txt")
    glob = np.float32(3.3424014e-05)
    codes = np.zeros((256, 8), np.uint8)
    scales = np.zeros((256, 1), np.uint8)
    for s in range(256):
        scales[s, 0] = s if s not in (0x7F, 0xFF) else 0
        for j in range(8):
            codes[s, j] = (2 * j) | ((2 * j + 1) << 4)
    got = oracle.dequant_f32(codes, scales, float(glob))
    other_order_differs = 0
    for s in range(256):
        sv = oracle.e4m3(int(scales[s, 0]))
        for c in range(16):
            exact = np.float64(e2[c]) * np.float64(sv) * np.float64(glob)
            assert got[s, c] == np.float32(exact)
            # rounding e4m3 * global to fp32 first double-rounds for some codes
            alt = np.float32(np.float32(e2[c]) * np.float32(np.float32(sv) * glob))
            other_order_differs += int(alt != got[s, c])
    assert other_order_differs > 0


def test_quantiser_round_trip_on_grid_values():
    """A tensor whose entries are already E2M1 * E4M3 * global (global 1) packs and
    decodes back to itself exactly."""
    rng = np.random.default_rng(0)
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rows, cols = 8, 64
    w = np.zeros((rows, cols))
    for r in range(rows):
        for b in range(cols // 16):
            sc = 2.0 ** rng.integers(-3, 5)
            blk = rng.choice(e2, 16) * rng.choice([-1, 1], 16) * sc
            blk[rng.integers(0, 16)] = 6 * sc                  # block amax on the grid top
            w[r, b * 16:(b + 1) * 16] = blk
    w[0, :16] = 0.0
    w[0, 0] = 2688.0                                             # tensor amax -> global 1
    bits = f32_to_bf16_bits_exact(w)
    codes, scales, g = testgen.quantize_nvfp4(bits)
    assert g == 1.0
    back = oracle.dequant_f64(codes, scales, g)
    np.testing.assert_array_equal(back, w)


def test_packer_scale_and_code_bounds_on_random_tensor():
    w = testgen.normal_bf16(7, 0, 0, 1, 0.02, 512 * 2048).reshape(512, 2048)
    codes, scales, g = testgen.quantize_nvfp4(w)
    wf = bf16_bits_to_f32(w).astype(np.float64)
    assert g == np.float32(np.float32(np.abs(wf).max()) / np.float32(2688.0))
    assert scales.max() == 0x7E                                  # the amax block gets 448
    assert not np.any((scales & 0x7F) == 0x7F)                   # never NaN
    back = oracle.dequant_f64(codes, scales, g)
    # NVFP4 error bound: half a grid step of the block's scale, at most
    # (6-4)/2 = 1 unit of s*global per element, plus the E4M3 rounding of s.
    blockmax = np.abs(wf).reshape(512, 128, 16).max(-1, keepdims=True)
    err = np.abs(back - wf).reshape(512, 128, 16)
    assert np.all(err <= blockmax / 6 * 1.0625 + 1e-12)
    rel = np.linalg.norm(back - wf) / np.linalg.norm(wf)
    assert 0.05 < rel < 0.15                                     # the usual NVFP4 error on N(0, s)
