"""GPU parity of the decode path (B = 1..8) against the fp64 oracle, through
the C ABI.  Inputs: the seeded synthetic Flint-shaped layer (hidden 2048, 256
routed experts + 1 shared, top-6, expert intermediate 512), x ~ N(0, 1) bf16,
weights ~ N(0, 0.02) bf16, packed to NVFP4 or kept bf16."""
import functools

import numpy as np
import pytest

import oracle
import testgen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")


@functools.lru_cache(maxsize=None)
def host_layer(seed: int, fmt: str = "nvfp4"):
    return testgen.make_layer(seed, 0, fmt)


_DEV = {}


def dev_layer(seed: int, fmt: str = "nvfp4"):
    key = (seed, fmt)
    if key not in _DEV:
        if len(_DEV) >= 3:                       # keep HBM use bounded
            _DEV.pop(next(iter(_DEV)))
        _DEV[key] = moe.DeviceLayer.from_host(host_layer(seed, fmt))
    return _DEV[key]


def run_forward(seed, B, fmt="nvfp4", x=None, ws=None):
    L = dev_layer(seed, fmt)
    if x is None:
        x = testgen.make_x(seed, B)
    xd = moe.device.to_device_bf16(x)
    out = torch.empty((B, 2048), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((B, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((B, 6), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, fmt=fmt))
    moe.moe_decode_forward(xd, L.router, L.routed, L.shared, out, ws, ids, w, fmt=fmt)
    torch.cuda.synchronize()
    return x, parity.bf16_out_to_f64(out), ids.cpu().numpy(), w.cpu().numpy()


def check_against_oracle(seed, B, fmt="nvfp4"):
    x, y, ids, w = run_forward(seed, B, fmt)
    HL = host_layer(seed, fmt)
    y_or, ids_or, w_or, gap = oracle.forward_layer(x, HL)
    log = []
    y_ref = parity.resolve_near_ties(x, HL, ids, y_or, ids_or, w_or, gap, log)
    parity.check_weights(ids, w, ids_or, w_or, gap)
    stats = parity.check_output(y, y_ref, f"seed {seed} B {B} {fmt}")
    if log:
        print(f"near-ties seed {seed} B {B}: {log}")
    return stats


# ----------------------------------------------------------------- dequant probe
def test_dequant_probe_bit_exact_all_tensors_of_a_layer():
    """Every one of the 771 NVFP4 tensors of a layer (257 experts x gate, up,
    down) decoded on the GPU equals the oracle's fp32(e2m1 * e4m3 * global)."""
    HL = host_layer(1)
    L = dev_layer(1)
    out_gu = torch.empty((512, 2048), dtype=torch.float32, device="cuda")
    out_d = torch.empty((2048, 512), dtype=torch.float32, device="cuda")
    for set_name, hx, dx in [("routed", HL.routed, L.routed), ("shared", HL.shared, L.shared)]:
        for e in range(hx.n):
            for t in range(3):
                o = out_gu if t < 2 else out_d
                moe.moe_nvfp4_dequant(dx, e, t, o)
                got = o.cpu().numpy()
                if t < 2:
                    want = oracle.dequant_f32(hx.w13[e, t], hx.w13_scale[e, t], float(hx.glob[e, t]))
                else:
                    want = oracle.dequant_f32(hx.w2[e], hx.w2_scale[e], float(hx.glob[e, 2]))
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (set_name, e, t)


def test_dequant_probe_covers_every_code_and_scale():
    """A synthetic tensor holding all 16 codes under all 254 finite scale bytes."""
    rows, cols = 512, 2048
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    scales = np.resize(scales, (rows, cols // 16)).copy()
    glob = np.float32(3.1e-5)

    class S:  # one-expert set with only the gate tensor meaningful
        fmt = "nvfp4"
    d = S()
    d.w13 = torch.from_numpy(np.stack([codes, codes])[None].copy()).cuda()
    d.w13_scale = torch.from_numpy(np.stack([scales, scales])[None].copy()).cuda()
    d.w2 = torch.zeros((1, 2048, 256), dtype=torch.uint8, device="cuda")
    d.w2_scale = torch.zeros((1, 2048, 32), dtype=torch.uint8, device="cuda")
    d.glob = torch.tensor([[glob, glob, glob]], dtype=torch.float32, device="cuda")
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    moe.moe_nvfp4_dequant(d, 0, 0, out)
    want = oracle.dequant_f32(codes, scales, float(glob))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ----------------------------------------------------------------- routing
@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("B", [1, 8])
def test_route_matches_oracle(seed, B):
    L = dev_layer(seed)
    x = testgen.make_x(seed, B)
    xd = moe.device.to_device_bf16(x)
    ids = torch.empty((B, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((B, 6), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))
    moe.moe_decode_route(xd, L.router, ids, w, ws)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    ids_or, w_or, gap, scores = oracle.route(x, host_layer(seed).router, 6)
    for t in range(B):
        if set(ids[t].tolist()) != set(ids_or[t].tolist()):
            assert gap[t] < parity.NEAR_TIE, (t, ids[t], ids_or[t], gap[t])
            continue
        # descending score order wherever the oracle's scores are apart
        s = scores[t][ids[t]]
        assert np.all(np.diff(s) < 1e-6)
    parity.check_weights(ids, w, ids_or, w_or, gap)


def test_route_zero_input_ties_to_lowest_indices():
    L = dev_layer(1)
    xd = torch.zeros((2, 2048), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((2, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((2, 6), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(2))
    moe.moe_decode_route(xd, L.router, ids, w, ws)
    torch.cuda.synchronize()
    assert ids.cpu().numpy().tolist() == [[0, 1, 2, 3, 4, 5]] * 2
    np.testing.assert_array_equal(w.cpu().numpy(), np.full((2, 6), 1 / 6, np.float32))


# ----------------------------------------------------------------- forward
@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_forward_b1_nvfp4(seed):
    check_against_oracle(seed, 1, "nvfp4")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_forward_b8_nvfp4(seed):
    check_against_oracle(seed, 8, "nvfp4")


@pytest.mark.parametrize("B", [2, 3, 4, 5, 6, 7])
def test_forward_every_batch_size(B):
    check_against_oracle(1, B, "nvfp4")


@pytest.mark.parametrize("seed,B", [(1, 1), (2, 1), (1, 8), (2, 8)])
def test_forward_bf16_weights(seed, B):
    check_against_oracle(seed, B, "bf16")


def test_batch_rows_match_single_token_calls():
    x, y8, ids8, _ = run_forward(2, 8)
    for t in range(8):
        _, y1, ids1, _ = run_forward(2, 1, x=x[t:t + 1].copy())
        np.testing.assert_array_equal(ids1[0], ids8[t])
        err = np.abs(y1[0] - y8[t]).max()
        assert err <= 2 ** -7 * max(1.0, np.abs(y1[0]).max()), err


def test_repeated_calls_are_bitwise_identical_and_reuse_the_workspace():
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(8))
    outs = [run_forward(3, B, ws=ws) for B in (8, 1, 8, 8)]
    np.testing.assert_array_equal(outs[0][1], outs[2][1])
    np.testing.assert_array_equal(outs[0][1], outs[3][1])
    x1, y1, _, _ = run_forward(3, 1)
    np.testing.assert_array_equal(outs[1][1], y1)


def test_identical_tokens_share_experts():
    """Eight copies of one token: each token's row equals the B = 1 result."""
    x = np.repeat(testgen.make_x(4, 1), 8, 0)
    _, y8, ids8, _ = run_forward(4, 8, x=x)
    _, y1, ids1, _ = run_forward(4, 1, x=x[:1].copy())
    for t in range(8):
        np.testing.assert_array_equal(ids8[t], ids1[0])
        np.testing.assert_array_equal(y8[t], y1[0])


def test_fused_and_split_paths_agree(monkeypatch):
    """The single-launch kernel and the three-launch path compute the same layer."""
    for B in (1, 3, 8):
        x, yf, idsf, wf = run_forward(5, B)
        monkeypatch.setenv("MOE_DECODE_SPLIT", "1")
        _, ys, idss, ws_ = run_forward(5, B, x=x)
        monkeypatch.delenv("MOE_DECODE_SPLIT")
        np.testing.assert_array_equal(idsf, idss)
        np.testing.assert_allclose(wf, ws_, rtol=1e-6)
        assert np.abs(yf - ys).max() <= 2 ** -7 * max(1.0, np.abs(ys).max())


def test_timed_entry_point_matches_and_times_the_kernel():
    """The timed variant computes the same layer and records a positive kernel
    duration on the caller's events."""
    L = dev_layer(2)
    for B in (1, 8):
        x = testgen.make_x(6, B)
        xd = moe.device.to_device_bf16(x)
        outs = [torch.empty((B, 2048), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))
        moe.moe_decode_forward(xd, L.router, L.routed, L.shared, outs[0], ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        moe.moe_decode_forward_timed(xd, L.router, L.routed, L.shared, outs[1], ws, e0, e1)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        ms = e0.elapsed_time(e1)
        assert 0.0 < ms < 50.0, ms


def test_layer_stack_in_a_hip_graph_matches_eager_and_oracle():
    """A stack of distinct layers captured in one HIP graph (the 47-layer
    configuration, here 4 layers): every replay, with eager work between
    replays, equals the eager pass bit for bit, and each layer matches the
    oracle."""
    nl, B = 4, 1
    host = [testgen.make_layer(1, l, "nvfp4") for l in range(nl)]
    dev = [moe.DeviceLayer.from_host(h) for h in host]
    x = testgen.make_x(21, B)
    xd = moe.device.to_device_bf16(x)
    outs = torch.empty((nl, B, 2048), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((nl, B, 6), dtype=torch.int32, device="cuda")
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))

    def one_pass():
        for l, d in enumerate(dev):
            moe.moe_decode_forward(xd, d.router, d.routed, d.shared, outs[l], ws, ids[l])

    one_pass()
    torch.cuda.synchronize()
    eager = outs.clone()
    ids_h = ids.cpu().numpy()
    for l in range(nl):
        y_or, ids_or, w_or, gap = oracle.forward_layer(x, host[l])
        y_ref = parity.resolve_near_ties(x, host[l], ids_h[l], y_or, ids_or, w_or, gap, [])
        parity.check_output(parity.bf16_out_to_f64(eager[l]), y_ref, f"stack layer {l}")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            one_pass()
    torch.cuda.synchronize()
    for rep in range(3):
        outs.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, eager), f"replay {rep}"
        one_pass()                                   # eager work between replays
        torch.cuda.synchronize()
    assert int(ws[8:12].view(torch.int32).item()) == 0


def test_workspace_error_word_stays_clear():
    """Byte offset 8 of the workspace is the device-side wait time-out flag."""
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(8))
    for B in (1, 8, 2):
        run_forward(1, B, ws=ws)
    assert int(ws[8:12].view(torch.int32).item()) == 0


def test_alternating_layers_share_one_workspace():
    """Calls on different layers, back to back on one stream and one workspace,
    each checked against the oracle: no value of one call leaks into the next."""
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(8))
    xs = {s: testgen.make_x(10 + s, 8) for s in (1, 2)}
    outs = []
    for rep in range(3):
        for seed in (1, 2):
            L = dev_layer(seed)
            xd = moe.device.to_device_bf16(xs[seed])
            out = torch.empty((8, 2048), dtype=torch.bfloat16, device="cuda")
            ids = torch.empty((8, 6), dtype=torch.int32, device="cuda")
            moe.moe_decode_forward(xd, L.router, L.routed, L.shared, out, ws, ids)
            outs.append((seed, out, ids))
    torch.cuda.synchronize()
    ref = {}
    for seed, out, ids in outs:
        y = parity.bf16_out_to_f64(out)
        if seed not in ref:
            HL = host_layer(seed)
            y_or, ids_or, w_or, gap = oracle.forward_layer(xs[seed], HL)
            y_ref = parity.resolve_near_ties(xs[seed], HL, ids.cpu().numpy(), y_or, ids_or, w_or,
                                             gap, [])
            parity.check_output(y, y_ref, f"seed {seed}")
            ref[seed] = y
        else:
            np.testing.assert_array_equal(y, ref[seed])
    assert int(ws[8:12].view(torch.int32).item()) == 0
