"""GPU parity of the general-shape decode path against the fp64 oracle,
through the C ABI: the other MoE shapes the pages name and the MXFP8 expert
format (the AREX article on vLLM's Day-0 support for Inkling-2-Small,
48-layer MoE section: Inkling's 256 experts, top-6 and two shared experts;
Inkling-2-Small's 384 experts, top-8 and none, MXFP8 experts in its last
layers), plus ragged shapes that exercise every lane split.

Inputs: seeded synthetic layers as for Flint (weights N(0, 0.02) bf16 packed
to the format, x ~ N(0, 1) bf16).  The pages give no hidden or expert
intermediate size for those models, so the named shapes keep Flint's 2048 and
512."""
import functools

import numpy as np
import pytest

import oracle
import testgen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")

# name: (H, I, E, K, n_shared, fmt)
SHAPES = {
    "inkling_nvfp4": (2048, 512, 256, 6, 2, "nvfp4"),
    "inkling2small_mxfp8": (2048, 512, 384, 8, 0, "mxfp8"),
    "inkling2small_nvfp4": (2048, 512, 384, 8, 0, "nvfp4"),
    "flint_mxfp8": (2048, 512, 256, 6, 1, "mxfp8"),
    "ragged_bf16": (1056, 96, 40, 3, 1, "bf16"),
    "wide_nvfp4": (4096, 1024, 128, 4, 1, "nvfp4"),
    "long_inter_mxfp8": (512, 2560, 64, 2, 0, "mxfp8"),
}


@functools.lru_cache(maxsize=2)
def layers(name: str, seed: int):
    H, I, E, K, NS, fmt = SHAPES[name]
    host = testgen.make_layer(seed, 0, fmt, H, I, E, K, n_shared=NS)
    return host, moe.DeviceLayer.from_host(host)


def S_of(name):
    H, I, E, K, NS, fmt = SHAPES[name]
    return moe.shape(moe._fmt(fmt), hidden=H, inter=I, n_experts=E, top_k=K, n_shared=NS)


def run(name, seed, B):
    H, I, E, K, NS, fmt = SHAPES[name]
    host, dl = layers(name, seed)
    S = S_of(name)
    x = testgen.make_x(seed + 100 * B, B, H)
    out = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
    w = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, S=S))
    moe.moe_decode_forward(moe.device.to_device_bf16(x), dl.router, dl.routed, dl.shared, out,
                           ws, ids, w, S=S)
    torch.cuda.synchronize()
    return host, x, parity.bf16_out_to_f64(out), ids.cpu().numpy(), w.cpu().numpy()


def check(name, seed, B):
    host, x, y, ids, w = run(name, seed, B)
    y_or, ids_or, w_or, gap = oracle.forward_layer(x, host)
    log = []
    y_ref = parity.resolve_near_ties(x, host, ids, y_or, ids_or, w_or, gap, log)
    parity.check_weights(ids, w, ids_or, w_or, gap)
    stats = parity.check_output(y, y_ref, f"{name} seed {seed} B {B}")
    if log:
        print(f"near-ties {name} B {B}: {log}")
    return stats


@pytest.mark.parametrize("B", [1, 8])
def test_inkling_two_shared_experts(B):
    check("inkling_nvfp4", 1, B)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_inkling2small_mxfp8(B):
    check("inkling2small_mxfp8", 2, B)


def test_inkling2small_nvfp4():
    check("inkling2small_nvfp4", 3, 2)


@pytest.mark.parametrize("B", [1, 8])
def test_flint_shape_in_mxfp8(B):
    check("flint_mxfp8", 4, B)


@pytest.mark.parametrize("name,B", [("ragged_bf16", 5), ("wide_nvfp4", 4),
                                    ("long_inter_mxfp8", 2), ("long_inter_mxfp8", 7)])
def test_ragged_and_wide_shapes(name, B):
    check(name, 5, B)


def test_route_only_on_a_general_shape():
    name = "inkling2small_mxfp8"
    H, I, E, K, NS, fmt = SHAPES[name]
    host, dl = layers(name, 2)
    S = S_of(name)
    B = 6
    x = testgen.make_x(77, B, H)
    ids = torch.empty((B, K), dtype=torch.int32, device="cuda")
    w = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, S=S))
    moe.moe_decode_route(moe.device.to_device_bf16(x), dl.router, ids, w, ws, S=S)
    torch.cuda.synchronize()
    ids_or, w_or, gap = oracle.route(x, host.router, K)[:3]
    parity.check_weights(ids.cpu().numpy(), w.cpu().numpy(), ids_or, w_or, gap)
    for t in range(B):
        if gap[t] >= parity.NEAR_TIE:
            assert ids.cpu().numpy()[t].tolist() == ids_or[t].tolist()   # descending score


def test_rows_of_a_batch_equal_single_token_calls():
    """Per-token independence on the general path, bit for bit."""
    name = "inkling_nvfp4"
    H = SHAPES[name][0]
    host, dl = layers(name, 1)
    S = S_of(name)
    x = testgen.make_x(91, 5, H)
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(5, S=S))
    out5 = torch.empty((5, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_decode_forward(moe.device.to_device_bf16(x), dl.router, dl.routed, dl.shared, out5,
                           ws, S=S)
    for t in range(5):
        o1 = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_forward(moe.device.to_device_bf16(x[t:t + 1].copy()), dl.router,
                               dl.routed, dl.shared, o1, ws, S=S)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out5[t]), t


def test_timed_entry_on_a_general_shape():
    name = "flint_mxfp8"
    H = SHAPES[name][0]
    host, dl = layers(name, 4)
    S = S_of(name)
    x = moe.device.to_device_bf16(testgen.make_x(92, 2, H))
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(2, S=S))
    a = torch.empty((2, H), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    moe.moe_decode_forward(x, dl.router, dl.routed, dl.shared, a, ws, S=S)
    moe.moe_decode_forward_timed(x, dl.router, dl.routed, dl.shared, b, ws, e0, e1, S=S)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and e0.elapsed_time(e1) > 0


def test_one_workspace_serves_the_general_and_the_flint_path():
    """The general path keeps to its own part of the workspace: Flint-shape
    and general-shape calls alternating on one workspace give the results of
    separate workspaces, bit for bit."""
    name = "inkling2small_mxfp8"
    H = SHAPES[name][0]
    _, dl = layers(name, 2)
    S = S_of(name)
    flint = moe.DeviceLayer.from_host(testgen.make_layer(1, 0, "nvfp4"))
    x = moe.device.to_device_bf16(testgen.make_x(93, 3, H))
    nbytes = max(moe.moe_workspace_bytes(3, S=S), moe.moe_workspace_bytes(3))
    shared_ws = moe.alloc_workspace(nbytes)

    def gen(ws):
        o = torch.empty((3, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_forward(x, dl.router, dl.routed, dl.shared, o, ws, S=S)
        return o

    def fl(ws):
        o = torch.empty((3, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_forward(x, flint.router, flint.routed, flint.shared, o, ws)
        return o
    ref_g = gen(moe.alloc_workspace(nbytes))
    ref_f = fl(moe.alloc_workspace(nbytes))
    outs = [fl(shared_ws), gen(shared_ws), fl(shared_ws), gen(shared_ws), fl(shared_ws)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref_f if i % 2 == 0 else ref_g), i


# ---------------------------------------------------------------- two shared experts
# Flint's shape with two shared experts (Inkling's) runs on the single-launch
# kernel; MOE_DECODE_SPLIT=1 sends it to the four-launch general path instead.

@pytest.mark.gpu
@pytest.mark.parametrize("B", [2, 3, 4, 5, 6, 7])
def test_inkling_single_launch_every_batch_size(B):
    check("inkling_nvfp4", 6, B)


@pytest.mark.gpu
def test_inkling_single_launch_agrees_with_the_general_path(monkeypatch):
    name = "inkling_nvfp4"
    H = SHAPES[name][0]
    host, dl = layers(name, 7)
    S = S_of(name)
    for B in (1, 8):
        x = testgen.make_x(94 + B, B, H)
        xd = moe.device.to_device_bf16(x)
        ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, S=S))
        outs = {}
        for split in ("0", "1"):
            monkeypatch.setenv("MOE_DECODE_SPLIT", split)
            o = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
            ids = torch.empty((B, 6), dtype=torch.int32, device="cuda")
            moe.moe_decode_forward(xd, dl.router, dl.routed, dl.shared, o, ws, ids_out=ids, S=S)
            torch.cuda.synchronize()
            outs[split] = (parity.bf16_out_to_f64(o), ids.cpu().numpy())
        y_or, ids_or, w_or, gap = oracle.forward_layer(x, host)
        for split, (y, ids) in outs.items():
            log = []
            y_ref = parity.resolve_near_ties(x, host, ids, y_or, ids_or, w_or, gap, log)
            parity.check_output(y, y_ref, f"{name} B {B} split {split}")
        # the two paths sum in different orders: equal ids, outputs within the parity bar
        confident = gap >= parity.NEAR_TIE
        for t in np.nonzero(confident)[0]:
            assert sorted(outs["0"][1][t]) == sorted(outs["1"][1][t]), t


@pytest.mark.gpu
def test_inkling_and_flint_single_launch_calls_share_a_workspace():
    """The two-shared-expert kernel and Flint's one-shared-expert kernel keep
    the same epoch counters and tagged slots: alternating calls on one
    workspace give the results of separate workspaces, bit for bit."""
    name = "inkling_nvfp4"
    H = SHAPES[name][0]
    _, dl = layers(name, 8)
    S = S_of(name)
    flint = moe.DeviceLayer.from_host(testgen.make_layer(2, 0, "nvfp4"))
    for B in (1, 4):
        x = moe.device.to_device_bf16(testgen.make_x(120 + B, B, H))
        nbytes = max(moe.moe_workspace_bytes(B, S=S), moe.moe_workspace_bytes(B))
        shared_ws = moe.alloc_workspace(nbytes)

        def ink(ws):
            o = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
            moe.moe_decode_forward(x, dl.router, dl.routed, dl.shared, o, ws, S=S)
            return o

        def fl(ws):
            o = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
            moe.moe_decode_forward(x, flint.router, flint.routed, flint.shared, o, ws)
            return o
        ref_i = ink(moe.alloc_workspace(nbytes))
        ref_f = fl(moe.alloc_workspace(nbytes))
        outs = [ink(shared_ws), fl(shared_ws), ink(shared_ws), ink(shared_ws), fl(shared_ws)]
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, ref_f if i in (1, 4) else ref_i), (B, i)
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        moe.moe_workspace_status(shared_ws, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
