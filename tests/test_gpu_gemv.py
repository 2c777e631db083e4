"""GPU parity of the dense NVFP4 GEMV (the non-expert projections) against the
fp64 oracle, through the C ABI.  Shapes: the attention projections of the
Flint shape (hidden 2048; 32 query and 4 key/value heads of 128, so a fused
q/k/v of 5120 rows and an output projection of 2048 x 4096), plus ragged and
minimal ones; weights N(0, 0.02) bf16 packed to NVFP4, x ~ N(0, 1) bf16."""
import numpy as np
import pytest

import oracle
import testgen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("moe_decode_sigmoid_amd")


def run(N, K, B, seed=1):
    codes, scales, glob = testgen.make_dense(seed, 0, N % 97, N, K)
    x = testgen.make_x(seed + K, B, K)
    dc = torch.from_numpy(codes).cuda()
    ds = torch.from_numpy(scales).cuda()
    dg = torch.tensor([glob], dtype=torch.float32, device="cuda")
    xd = moe.device.to_device_bf16(x)
    y = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    moe.moe_nvfp4_gemv(xd, dc, ds, dg, y)
    torch.cuda.synchronize()
    return parity.bf16_out_to_f64(y), oracle.gemv_nvfp4(x, codes, scales, glob)


def check(y, ref, what):
    """Rounding y once to bf16 costs at most 2^-9 |y|; fp32 accumulation far less."""
    err = np.abs(y - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * np.sqrt(np.mean(ref ** 2))
    assert np.all(err <= bound), f"{what}: worst excess {np.max(err - bound):.3e}"
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 5e-3, f"{what}: rel L2 {rel:.3e}"


@pytest.mark.parametrize("N,K,B", [
    (5120, 2048, 1), (5120, 2048, 8), (2048, 4096, 1), (2048, 4096, 8),
    (37, 96, 3), (1, 32, 1), (300, 8192, 4), (1000, 2080, 2), (16, 2048, 5)])
def test_gemv_matches_oracle(N, K, B):
    y, ref = run(N, K, B)
    check(y, ref, f"N {N} K {K} B {B}")


def test_gemv_rows_match_single_token_calls():
    """Token t of a batch equals the same token alone, bit for bit."""
    N, K = 512, 2048
    codes, scales, glob = testgen.make_dense(3, 0, 1, N, K)
    x = testgen.make_x(4, 6, K)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    dg = torch.tensor([glob], dtype=torch.float32, device="cuda")
    y6 = torch.empty((6, N), dtype=torch.bfloat16, device="cuda")
    moe.moe_nvfp4_gemv(moe.device.to_device_bf16(x), dc, ds, dg, y6)
    for t in range(6):
        y1 = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
        moe.moe_nvfp4_gemv(moe.device.to_device_bf16(x[t:t + 1].copy()), dc, ds, dg, y1)
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y6[t]), t


def test_gemv_zero_input_gives_zero():
    N, K = 64, 1024
    codes, scales, glob = testgen.make_dense(5, 0, 2, N, K)
    y = torch.full((2, N), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_nvfp4_gemv(torch.zeros((2, K), dtype=torch.bfloat16, device="cuda"),
                       torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                       torch.tensor([glob], dtype=torch.float32, device="cuda"), y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
