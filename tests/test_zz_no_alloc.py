"""GPU test of moe_decode_forward_noalloc (the decode layer on the library's
own per-GPU scratch array, for callers that cannot allocate), through the C
ABI: two calls in a row, the second with a smaller batch, each bit-equal to
moe_decode_forward on a fresh workspace (the same kernels), and both within
the layer's tolerance of the fp64 oracle.  Inputs: the seeded synthetic
Flint-shaped NVFP4 and BF16 layers of the decode tests."""
import functools

import pytest

import oracle
import testgen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")


@functools.lru_cache(maxsize=2)
def layer(fmt: str):
    host = testgen.make_layer(41, 0, fmt)
    return host, moe.DeviceLayer.from_host(host)


def run_both(fmt, B, seed):
    host, d = layer(fmt)
    x = testgen.make_x(seed, B)
    xd = moe.device.to_device_bf16(x)
    out_n = torch.empty((B, 2048), dtype=torch.bfloat16, device="cuda")
    ids_n = torch.empty((B, 6), dtype=torch.int32, device="cuda")
    w_n = torch.empty((B, 6), dtype=torch.float32, device="cuda")
    moe.moe_decode_forward_noalloc(xd, d.router, d.routed, d.shared, out_n, ids_n, w_n, fmt=fmt)
    out_r = torch.empty_like(out_n)
    ids_r = torch.empty_like(ids_n)
    w_r = torch.empty_like(w_n)
    ws = moe.alloc_workspace(moe.moe_workspace_bytes(B, fmt=fmt))
    moe.moe_decode_forward(xd, d.router, d.routed, d.shared, out_r, ws, ids_r, w_r, fmt=fmt)
    torch.cuda.synchronize()
    return host, x, out_n, ids_n, w_n, out_r, ids_r, w_r


@pytest.mark.parametrize("fmt", ["nvfp4", "bf16"])
def test_noalloc_matches_the_workspace_entry_point_twice(fmt):
    for B, seed in ((8, 301), (3, 302)):            # the second call is smaller
        print(f"noalloc {fmt} B={B}", flush=True)
        host, x, out_n, ids_n, w_n, out_r, ids_r, w_r = run_both(fmt, B, seed)
        assert torch.equal(ids_n, ids_r)
        assert torch.equal(w_n, w_r)
        assert torch.equal(out_n, out_r)
        y_or, ids_or, w_or, gap = oracle.forward_layer(x, host)
        log = []
        y_ref = parity.resolve_near_ties(x, host, ids_n.cpu().numpy(), y_or, ids_or, w_or, gap,
                                         log)
        parity.check_output(parity.bf16_out_to_f64(out_n), y_ref, f"noalloc {fmt} B {B}")


def test_noalloc_rejects_what_its_array_cannot_hold():
    host, d = layer("nvfp4")
    x = moe.device.to_device_bf16(testgen.make_x(303, 9))
    out = torch.empty((9, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_forward_noalloc(x, d.router, d.routed, d.shared, out)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    S = moe.shape(moe.MOE_W_NVFP4, n_experts=384, top_k=8, n_shared=0)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_forward_noalloc(x[:2], d.router, d.routed, None, out[:2], S=S)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
