"""GPU tests of the stacked decode entry (a stack of independent layers in one
launch): each layer of the stack must equal moe_decode_forward on that layer
bit for bit (same kernel code), and the oracle within tolerance; a HIP graph
of the stack replays to the same bits.  Inputs: the seeded synthetic
Flint-shaped layers of the decode tests."""
import numpy as np
import pytest

import oracle
import testgen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")

_CACHE = {}


def stack(fmt: str, L: int = 5, seed: int = 11):
    key = (fmt, L, seed)
    if key not in _CACHE:
        _CACHE.clear()
        hosts = [testgen.make_layer(seed, l, fmt) for l in range(L)]
        devs = [moe.DeviceLayer.from_host(h) for h in hosts]
        _CACHE[key] = (hosts, devs, moe.layer_table(devs))
    return _CACHE[key]


def run_both(fmt, B, L=5):
    hosts, devs, table = stack(fmt, L)
    x = testgen.make_x(50 + B, B)
    xd = moe.device.to_device_bf16(x)
    S = moe.shape(moe._fmt(fmt))
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, fmt=fmt))
    out_s = torch.empty((L, B, 2048), dtype=torch.bfloat16, device="cuda")
    ids_s = torch.empty((L, B, 6), dtype=torch.int32, device="cuda")
    moe.moe_decode_stack_forward(xd, table, out_s, ws, ids_s, S=S)
    out_1 = torch.empty_like(out_s)
    ids_1 = torch.empty_like(ids_s)
    for l, d in enumerate(devs):
        moe.moe_decode_forward(xd, d.router, d.routed, d.shared, out_1[l], ws, ids_1[l], S=S)
    torch.cuda.synchronize()
    return hosts, x, out_s, ids_s, out_1, ids_1


# The stacked launch issues the next layer's routing-independent rows right
# after the h copy when every routed down row is already in flight (NVFP4
# B <= 5) and behind the last down-row loads otherwise (NVFP4 B >= 6, BF16
# B >= 2): both sides of that boundary are covered.
@pytest.mark.parametrize("fmt,B", [("nvfp4", 1), ("nvfp4", 3), ("nvfp4", 5), ("nvfp4", 6),
                                   ("nvfp4", 8), ("bf16", 1), ("bf16", 2)])
def test_stack_equals_per_layer_calls_bitwise(fmt, B):
    hosts, x, out_s, ids_s, out_1, ids_1 = run_both(fmt, B)
    assert torch.equal(ids_s, ids_1)
    for l in range(out_s.shape[0]):
        assert torch.equal(out_s[l], out_1[l]), l


@pytest.mark.parametrize("B", [2, 8])
def test_stack_layers_match_the_oracle(B):
    hosts, x, out_s, ids_s, _, _ = run_both("nvfp4", B)
    for l in (0, 4):
        y_or, ids_or, w_or, gap = oracle.forward_layer(x, hosts[l])
        log = []
        ids = ids_s[l].cpu().numpy()
        y_ref = parity.resolve_near_ties(x, hosts[l], ids, y_or, ids_or, w_or, gap, log)
        parity.check_output(parity.bf16_out_to_f64(out_s[l]), y_ref, f"stack layer {l}")


def test_batch1_stack_after_launches_of_one_to_seven_workgroups():
    """At batch 1 the stacked launch exchanges the router logits inside each
    XCD.  The hardware deals a launch's workgroups out to the 8 XCDs in turn,
    starting where the previous dispatch stopped, so 1 .. 7 one-workgroup
    launches (the status kernel) before it change which workgroups share an
    XCD.  Every such start gives the same bits, and no wait gives up."""
    hosts, devs, table = stack("nvfp4")
    B = 1
    xd = moe.device.to_device_bf16(testgen.make_x(61, B))
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    out = torch.empty((len(devs), B, 2048), dtype=torch.bfloat16, device="cuda")
    moe.moe_decode_stack_forward(xd, table, out, ws)
    moe.moe_workspace_status(ws, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = out.clone()
    for shift in range(1, 8):
        print(f"batch-1 stack after {shift} one-workgroup launches", flush=True)
        out.zero_()
        torch.cuda.synchronize()
        for _ in range(shift):
            moe.moe_workspace_status(ws, st)
        moe.moe_decode_stack_forward(xd, table, out, ws)
        moe.moe_workspace_status(ws, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, (shift, int(st.item()))
        assert torch.equal(out, ref), shift


def test_stack_in_a_hip_graph_replays_to_the_same_bits():
    hosts, devs, table = stack("nvfp4")
    B = 1
    xd = moe.device.to_device_bf16(testgen.make_x(60, B))
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))
    out = torch.empty((len(devs), B, 2048), dtype=torch.bfloat16, device="cuda")
    moe.moe_decode_stack_forward(xd, table, out, ws)
    torch.cuda.synchronize()
    ref = out.clone()
    out.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_decode_stack_forward(xd, table, out, ws)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        # eager work between replays
        moe.moe_decode_forward(xd, devs[0].router, devs[0].routed, devs[0].shared, out[0], ws)
        torch.cuda.synchronize()
