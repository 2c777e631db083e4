"""GPU parity of the W4A4 decode layer (NVFP4 weights, NVFP4 activations with
the Four Over Six block scale: the AREX article on vLLM's Day-0 support for
Inkling-2-Small, 48-layer MoE section) against the fp64 oracle, through the
C ABI.

Both quantisations are decisions taken in fp32 (block scale 6 or 4, codes),
so they are compared bit for bit: the quantised x against the oracle's
quantiser on the same x, the quantised h against the oracle's quantiser on
the GPU's own h (read from the workspace through the documented diagnostic
offsets).  The GPU's h before quantisation is compared with the oracle's
within bf16 rounding, and the output with the oracle evaluated on the GPU's
h, at the usual tolerance (a decomposition).  End to end, the output is also
compared with the oracle run from x alone (its own quantised x, h and
quantised h) at the same tolerance, ids forced only for near-ties.  Inputs: seeded synthetic NVFP4 layers (weights
N(0, 0.02) bf16 packed to NVFP4, x ~ N(0, 1) bf16)."""
import contextlib
import os

import numpy as np
import pytest

import oracle
import testgen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")

# name: (H, I, E, K, n_shared)
SHAPES = {
    "flint": (2048, 512, 256, 6, 1),
    "inkling2small": (2048, 512, 384, 8, 0),
    "ragged": (1056, 96, 40, 3, 2),
}
_CACHE = {}


def layer(name, seed):
    if (name, seed) not in _CACHE:
        _CACHE.clear()
        H, I, E, K, NS = SHAPES[name]
        host = testgen.make_layer(seed, 0, "nvfp4", H, I, E, K, n_shared=NS)
        _CACHE[(name, seed)] = (host, moe.DeviceLayer.from_host(host))
    return _CACHE[(name, seed)]


def bf16_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@contextlib.contextmanager
def general_path(on=True):
    """Flint's shape at batch 1 runs on the single-launch kernel; with this
    switch (the library's MOE_DECODE_SPLIT) it takes the four-launch general
    path, whose workspace exposes x, h and their quantisations."""
    old = os.environ.get("MOE_DECODE_SPLIT")
    if on:
        os.environ["MOE_DECODE_SPLIT"] = "1"
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("MOE_DECODE_SPLIT", None)
        else:
            os.environ["MOE_DECODE_SPLIT"] = old


def run(name, seed, B, general=False):
    H, I, E, K, NS = SHAPES[name]
    host, dl = layer(name, seed)
    S = moe.shape(moe.MOE_W_NVFP4_A4, hidden=H, inter=I, n_experts=E, top_k=K, n_shared=NS)
    x = testgen.make_x(seed + 7 * B, B, H)
    out = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
    w = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, S=S))
    with general_path(general):
        moe.moe_decode_forward(moe.device.to_device_bf16(x), dl.router, dl.routed, dl.shared, out,
                               ws, ids, w, S=S)
        torch.cuda.synchronize()
    off = moe.general_workspace_layout(S)
    raw = ws.cpu().numpy()

    def arr(key, dtype, count):
        return raw[off[key]:off[key] + count * np.dtype(dtype).itemsize].view(dtype)
    na = int(arr("n_entries", np.int32, 1)[0])
    ws_d = dict(entry=arr("entry", np.int32, 66)[:na].copy(),
                amask=arr("amask", np.uint32, 66)[:na].copy(),
                h=arr("h", np.uint16, 66 * 8 * I).reshape(66, 8, I),
                xq=arr("xq", np.uint16, 8 * H).reshape(8, H), gx=arr("gx", np.float32, 8),
                hq=arr("hq", np.uint16, 66 * 8 * I).reshape(66, 8, I),
                gh=arr("gh", np.float32, 66 * 8).reshape(66, 8))
    return host, x, parity.bf16_out_to_f64(out), ids.cpu().numpy(), w.cpu().numpy(), ws_d


def slots_of(ws_d, B):
    """The GPU's h per (token, slot), slots in the oracle's order (routed ids
    ascending, then the shared experts), and the entry index of each."""
    out, idx = [], []
    for t in range(B):
        a_s = [a for a in range(len(ws_d["entry"])) if (ws_d["amask"][a] >> t) & 1]
        out.append(np.stack([ws_d["h"][a, t] for a in a_s]))
        idx.append(a_s)
    return np.stack(out), idx


@pytest.mark.parametrize("name,B", [("flint", 1), ("flint", 8), ("inkling2small", 3),
                                    ("ragged", 5)])
def test_w4a4_layer(name, B):
    host, x, y, ids, w, ws_d = run(name, 3, B, general=True)
    # 1. x quantised bit for bit as the oracle quantises it
    for t in range(B):
        codes, scales, g, vals = oracle.quant_fp4_46(bf16_f64(x[t]).astype(np.float32))
        assert np.float32(ws_d["gx"][t]) == np.float32(g), t
        np.testing.assert_array_equal(bf16_f64(ws_d["xq"][t]) * np.float64(np.float32(g)), vals)
    # 2. h before quantisation: the oracle's within bf16 rounding
    h_gpu, entries = slots_of(ws_d, B)
    y_or, ids_or, w_or, gap, h_or = oracle.forward_w4a4(x, host)
    same = [t for t in range(B) if set(ids[t].tolist()) == set(ids_or[t].tolist())]
    for t in range(B):
        if t not in same:
            assert gap[t] < parity.NEAR_TIE, (t, gap[t])
    hg, ho = bf16_f64(h_gpu[same]), bf16_f64(h_or[same])
    assert np.all(np.abs(hg - ho) <= 2.0 ** -7 * np.abs(ho) + 1e-6 * np.abs(ho).max())
    # 3. h quantised bit for bit as the oracle quantises the GPU's h
    for t in range(B):
        for s, a in enumerate(entries[t]):
            codes, scales, g, vals = oracle.quant_fp4_46(bf16_f64(h_gpu[t, s]).astype(np.float32))
            assert np.float32(ws_d["gh"][a, t]) == np.float32(g), (t, s)
            np.testing.assert_array_equal(bf16_f64(ws_d["hq"][a, t]) * np.float64(np.float32(g)),
                                          vals)
    # 4. the output against the oracle on the GPU's h (and ids, for logged near-ties)
    y_ref, ids_r, w_r, gap_r, _ = oracle.forward_w4a4(x, host, forced_ids=ids.copy(), h_in=h_gpu)
    parity.check_weights(ids, w, ids_or, w_or, gap)
    parity.check_output(y, y_ref, f"w4a4 {name} B {B}")


def test_w4a4_tokens_are_independent():
    """On the general path a token's result does not depend on the batch."""
    host, x, y, ids, w, _ = run("flint", 4, 4, general=True)
    H = SHAPES["flint"][0]
    host, dl = layer("flint", 4)
    S = moe.shape(moe.MOE_W_NVFP4_A4)
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(1, S=S))
    with general_path():
        for t in range(4):
            o = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
            moe.moe_decode_forward(moe.device.to_device_bf16(x[t:t + 1].copy()), dl.router,
                                   dl.routed, dl.shared, o, ws, S=S)
            torch.cuda.synchronize()
            assert np.array_equal(parity.bf16_out_to_f64(o)[0], y[t]), t


@pytest.mark.parametrize("name,B,seed", [("flint", 1, 5), ("flint", 8, 5), ("flint", 4, 6),
                                         ("inkling2small", 3, 5), ("ragged", 5, 5)])
def test_w4a4_end_to_end_against_the_oracles_own_h(name, B, seed):
    """The W4A4 output against the fp64 oracle run from x alone: its own
    quantised x, its own h, its own quantisation of h (no GPU value enters
    it).  ids are forced to the GPU's only for a token whose oracle 6th/7th
    score gap is below the near-tie threshold."""
    host, x, y, ids, w, _ = run(name, seed, B)
    y_or, ids_or, w_or, gap, _ = oracle.forward_w4a4(x, host)
    for t in range(B):
        if set(ids[t].tolist()) != set(ids_or[t].tolist()):
            assert gap[t] < parity.NEAR_TIE, (t, gap[t])
            print(f"token {t}: near-tie (gap {gap[t]:.2e}), ids forced")
            y_or[t] = oracle.forward_w4a4(x[t:t + 1].copy(), host,
                                          forced_ids=ids[t:t + 1].copy())[0][0]
    parity.check_weights(ids, w, ids_or, w_or, gap)
    print(parity.check_output(y, y_or, f"w4a4 e2e {name} B {B}"))


# ---------------------------------------------------------------- single launch
# Flint's shape at batch 1 to 8 runs on the single-launch kernel, every
# workgroup quantising x and all h pairs itself with the same decisions.

@pytest.mark.parametrize("B,seed", [(1, 11), (1, 12), (1, 13), (2, 14), (5, 15), (8, 16)])
def test_w4a4_single_launch_end_to_end(B, seed):
    test_w4a4_end_to_end_against_the_oracles_own_h("flint", B, seed)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_w4a4_single_launch_agrees_with_the_general_path(B):
    for seed in (21, 22):
        _, _, y1, ids1, w1, _ = run("flint", seed, B)
        _, _, y2, ids2, w2, _ = run("flint", seed, B, general=True)
        for t in range(B):
            assert sorted(ids1[t].tolist()) == sorted(ids2[t].tolist()), t
            np.testing.assert_allclose(np.sort(w1[t]), np.sort(w2[t]), rtol=2e-5, atol=1e-6)
        parity.check_output(y1, y2, f"w4a4 single launch vs general, B {B}, seed {seed}")


@pytest.mark.parametrize("B", [1, 8])
def test_w4a4_single_launch_repeats_and_shares_a_workspace(B):
    """Repeated calls give the same bits, and W4A4 and W4A16 single-launch
    calls alternate on one workspace as on separate ones."""
    H = SHAPES["flint"][0]
    host, dl = layer("flint", 31)
    S4 = moe.shape(moe.MOE_W_NVFP4_A4)
    x = moe.device.to_device_bf16(testgen.make_x(131, B, H))
    nbytes = max(moe.moe_workspace_bytes(B, S=S4), moe.moe_workspace_bytes(B))
    ws = moe.alloc_workspace(nbytes)

    def call(S):
        o = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_forward(x, dl.router, dl.routed, dl.shared, o, ws, S=S)
        return o
    ref4 = call(S4)
    ref16 = call(None)
    outs = [call(S4), call(None), call(S4), call(S4), call(None)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref16 if i in (1, 4) else ref4), i
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    moe.moe_workspace_status(ws, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0


@pytest.mark.gpu
def test_quantiser_converts_equal_the_rounding_definitions():
    """The single-launch quantiser's E4M3 and E2M1 roundings come from
    gfx950's fp32 -> FP8 / FP4 converts; over every fp32 bit pattern they
    equal the roundings written out as arithmetic (nearest-even, saturating
    at 448 and 6)."""
    counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    moe.moe_a4_convert_check(counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0]
