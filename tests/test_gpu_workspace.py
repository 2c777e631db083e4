"""GPU tests of the workspace contract (include/moe_decode.h):

1. One workspace serves every entry point: prefill, decode, the stacked and
   the chained launches alternate on it, and every result equals the same
   call on a fresh workspace bit for bit (the prefill data lies past the
   region where the single-launch decode kernels keep their call counters).
2. A wait that gives up is reported.  The time-out is forced from the host:
   the workspace is filled with the byte 0x01 instead of zeros, so every
   workgroup's call counter agrees (the logit exchange works) but the
   h-ready counters can never reach the value the call waits for.  Every
   wait is bounded, so the kernel ends; moe_workspace_status then reports
   the h hand-over bit (2) once and is clear on the next read.
3. Determinism soak: 2,000 replays of a 47-layer stacked pass and of a
   47-layer chained pass are each bit-equal to the first, with the wait
   status clear at the end.

Inputs: seeded synthetic Flint-shaped NVFP4 layers."""
import numpy as np
import pytest

import testgen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")

H = 2048
_DEV = {}


def layers(n: int, seed: int = 31):
    key = (n, seed)
    if key not in _DEV:
        _DEV.clear()
        torch.cuda.empty_cache()
        _DEV[key] = [moe.DeviceLayer.from_host(testgen.make_layer(seed, l)) for l in range(n)]
    return _DEV[key]


def status_of(ws) -> int:
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    moe.moe_workspace_status(ws, st)
    torch.cuda.synchronize()
    return int(st.item())


def test_one_workspace_serves_prefill_and_decode():
    print("shared workspace: prefill / decode / stack / chain", flush=True)
    ds = layers(3)
    d = ds[0]
    table = moe.layer_table(ds)
    T, B = 300, 4
    xp = moe.device.to_device_bf16(testgen.make_x(71, T))
    xd = moe.device.to_device_bf16(testgen.make_x(72, B))
    nwd = moe.device.to_device_bf16(testgen.make_x(73, 3))
    need = max(moe.moe_workspace_bytes(T, prefill=True), moe.moe_workspace_bytes(B))

    def prefill(ws):
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_prefill_forward(xp, d.router, d.routed, d.shared, y, ws)
        return y

    def decode(ws):
        y = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_forward(xd, d.router, d.routed, d.shared, y, ws)
        return y

    def stacked(ws):
        y = torch.empty((3, B, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_stack_forward(xd, table, y, ws)
        return y

    def chained(ws):
        y = torch.empty((3, B, H), dtype=torch.bfloat16, device="cuda")
        moe.moe_decode_chain_forward(xd, table, y, ws, norm_w=nwd, eps=1e-5)
        return y

    order = [prefill, decode, stacked, chained, prefill, decode, prefill, chained, decode]
    ws = moe.alloc_workspace(need)
    got = [f(ws) for f in order]
    torch.cuda.synchronize()
    for i, f in enumerate(order):
        alone = f(moe.alloc_workspace(need))        # the same call on a fresh workspace
        torch.cuda.synchronize()
        assert torch.equal(got[i], alone), (i, f.__name__)
    assert status_of(ws) == 0


def test_forced_wait_timeout_is_reported_and_cleared():
    print("forced h-ready time-out (workspace filled with 0x01)", flush=True)
    d = layers(3)[0]
    B = 2
    xd = moe.device.to_device_bf16(testgen.make_x(74, B))
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))
    assert status_of(ws) == 0
    ws.fill_(1)
    assert status_of(ws) == 0x01010101  # the fill pattern in the status word itself: cleared
    out = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_decode_forward(xd, d.router, d.routed, d.shared, out, ws)
    torch.cuda.synchronize()
    s1 = status_of(ws)
    assert s1 == 2, s1                 # the h hand-over gave up; the logit exchange did not
    assert status_of(ws) == 0          # read and cleared
    # a zeroed workspace again: the same call completes its hand-overs
    ws.zero_()
    moe.moe_decode_forward(xd, d.router, d.routed, d.shared, out, ws)
    torch.cuda.synchronize()
    assert status_of(ws) == 0


@pytest.mark.parametrize("kind", ["stack", "chain"])
def test_determinism_soak_2000_passes_of_47_layers(kind):
    """47 layers per pass (4 distinct layers, cycled in the layer table), one
    launch per pass captured in a HIP graph; every replay's output is compared
    with the first on the device, the mismatch count read every 250 replays."""
    print(f"soak: 2000 {kind} passes", flush=True)
    ds = layers(4)
    table = moe.layer_table([ds[l % 4] for l in range(47)])
    B = 1
    xd = moe.device.to_device_bf16(testgen.make_x(75, B))
    nwd = moe.device.to_device_bf16(testgen.make_x(76, 47))
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B))
    out = torch.empty((47, B, H), dtype=torch.bfloat16, device="cuda")

    def one():
        if kind == "stack":
            moe.moe_decode_stack_forward(xd, table, out, ws)
        else:
            moe.moe_decode_chain_forward(xd, table, out, ws, norm_w=nwd, eps=1e-5)
    one()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(2000):
        g.replay()
        bad += (out != ref).sum()
        if i % 250 == 249:
            n = int(bad.item())
            assert n == 0, f"replay {i}: {n} elements differ"
    assert status_of(ws) == 0
