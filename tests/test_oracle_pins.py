"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Layer definition ("Day-0 Support for Flint on vLLM", Model architecture:
256 experts chosen by a sigmoid top-6 plus one shared expert; Optimization,
Fig. 2 list: only the selected experts' weights are read; SiLU kernels;
low-latency path: routing and expert combine).  Each test below would fail for
a plausible slip in the oracle: a dropped or extra term, a wrong sign, a
swapped gate/up, a transposed matrix, a wrong tie order or expert index.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import testgen
from tests.helpers import bf16_bits_to_f32, f32_to_bf16_bits_exact, load_table

H, I, E, K = 32, 16, 8, 2


def tiny_layer(seed=3, fmt="nvfp4", H=H, I=I, E=E, K=K, sigma=0.5):
    return testgen.make_layer(seed, 0, fmt, H, I, E, K, sigma)


def f64(u16):
    return bf16_bits_to_f32(u16).astype(np.float64)


# ----------------------------------------------------------------- routing
def test_sigmoid_matches_library():
    for z in [-40.0, -3.0, -1e-3, 0.0, 0.5, 2.0, 30.0]:
        assert oracle.sigmoid(z) == pytest.approx(float(expit(z)), rel=1e-15, abs=1e-300)


def test_router_logits_match_numpy_gemv():
    x = testgen.make_x(5, 1, 2048)[0]
    R = testgen.make_router(5, 0)
    got = oracle.router_logits(x, R)
    want = f64(R) @ f64(x)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(20))
def test_topk_is_the_max_sum_subset(seed):
    """For distinct scores the top-k set is the unique k-subset of largest sum,
    found here by brute force over all C(E, k) subsets."""
    rng = np.random.default_rng(seed)
    n, k = 12, 4
    scores = expit(rng.normal(0, 1, n))
    ids, gap = oracle.topk(scores, k)
    best = max(itertools.combinations(range(n), k), key=lambda c: scores[list(c)].sum())
    assert sorted(ids.tolist()) == sorted(best)
    assert all(scores[ids[j]] > scores[ids[j + 1]] for j in range(k - 1))
    rest = sorted(set(range(n)) - set(ids.tolist()), key=lambda e: -scores[e])
    assert gap == scores[ids[-1]] - scores[rest[0]]


def test_zero_input_ties_pick_lowest_indices():
    """x = 0 -> every logit 0, every score 1/2 -> ids 0..5, w = 1/6."""
    x = np.zeros((1, 2048), np.uint16)
    R = testgen.make_router(1, 0)
    ids, w, gap, _ = oracle.route(x, R, 6)
    assert ids[0].tolist() == [0, 1, 2, 3, 4, 5]
    np.testing.assert_array_equal(w[0], np.full(6, 1 / 6))
    assert gap[0] == 0.0


def test_duplicate_router_rows_tie_to_lower_index():
    x = testgen.make_x(2, 1, 2048)
    R = testgen.make_router(2, 0).copy()
    logits = oracle.router_logits(x[0], R)
    top = int(np.argmax(logits))
    R[200] = R[top]                     # an exact duplicate of the best expert, higher index
    R[top if top < 100 else 0] = R[top]
    ids, _, _, _ = oracle.route(x, R, 6)
    dup = sorted({top, 200, top if top < 100 else 0})
    assert ids[0][:len(dup)].tolist() == dup


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_renormalised_weights(seed):
    x = testgen.make_x(seed, 4, 2048)
    R = testgen.make_router(seed, 0)
    ids, w, gap, scores = oracle.route(x, R, 6)
    logits = f64(x) @ f64(R).T
    for t in range(4):
        s = expit(logits[t])
        np.testing.assert_allclose(scores[t], s, rtol=1e-12)
        assert sorted(ids[t].tolist()) == sorted(np.argsort(-s, kind="stable")[:6].tolist())
        assert abs(w[t].sum() - 1.0) < 1e-15
        assert np.all((w[t] > 0) & (w[t] < 1))
        np.testing.assert_allclose(w[t], s[ids[t]] / s[ids[t]].sum(), rtol=1e-14)
        assert gap[t] > 0


# ----------------------------------------------------------------- experts
def _bf16_experts(w13, w2):
    """An expert set in bf16 format from float arrays (values must be bf16-exact)."""
    n = w13.shape[0]
    return testgen.Experts("bf16", n, f32_to_bf16_bits_exact(w13), f32_to_bf16_bits_exact(w2))


def _round_bf16(a):
    return bf16_bits_to_f32(np.array([testgen.bf16_rne(float(v)) for v in a.ravel()],
                                     np.uint16)).reshape(a.shape)


def test_expert_is_silu_gated_ffn_when_gate_saturates():
    """With every gate pre-activation g >= 60, SiLU(g) = g to 1e-26, so the
    expert reduces to D ((G x) * (U x)) — a plain matrix product checked with
    numpy.  A swapped gate/up, a transposed D or a dropped product fails."""
    rng = np.random.default_rng(0)
    x = np.abs(_round_bf16(rng.normal(0, 1, H))) + 0.25
    x = _round_bf16(x)
    G = _round_bf16(np.abs(rng.normal(0, 1, (I, H))) + 2.0)     # g = G x >> 0
    U = _round_bf16(rng.normal(0, 1, (I, H)))
    D = _round_bf16(rng.normal(0, 1, (H, I)))
    X = _bf16_experts(np.stack([G, U])[None], D[None])
    g = G.astype(np.float64) @ x
    assert g.min() > 60
    want = D.astype(np.float64) @ (g * (U.astype(np.float64) @ x))
    got = oracle.expert(X, 0, x.astype(np.float64), H, I)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13 * np.abs(want).max())


def test_expert_vanishes_when_gate_is_very_negative():
    rng = np.random.default_rng(1)
    x = _round_bf16(np.abs(rng.normal(0, 1, H)) + 0.25)
    G = _round_bf16(-(np.abs(rng.normal(0, 1, (I, H))) + 2.0))  # g << 0 -> SiLU(g) ~ g e^g
    U = _round_bf16(rng.normal(0, 1, (I, H)) * 50)
    D = _round_bf16(rng.normal(0, 1, (H, I)))
    X = _bf16_experts(np.stack([G, U])[None], D[None])
    got = oracle.expert(X, 0, x.astype(np.float64), H, I)
    assert np.abs(got).max() < 1e-20


def test_expert_at_zero_gate_is_zero():
    rng = np.random.default_rng(2)
    x = _round_bf16(rng.normal(0, 1, H))
    G = np.zeros((I, H), np.float32)
    U = _round_bf16(rng.normal(0, 1, (I, H)))
    D = _round_bf16(rng.normal(0, 1, (H, I)))
    X = _bf16_experts(np.stack([G, U])[None], D[None])
    got = oracle.expert(X, 0, x.astype(np.float64), H, I)
    assert np.all(got == 0)


def test_silu_value_at_ln3():
    """sigmoid(ln 3) = 3/4, so an expert with a single active path computes
    0.75 ln3 * u * d exactly up to rounding."""
    x = np.zeros(H, np.float32)
    x[0] = 1.0
    G = np.zeros((I, H), np.float32)
    U = np.zeros((I, H), np.float32)
    D = np.zeros((H, I), np.float32)
    ln3 = float(_round_bf16(np.array([np.log(3.0)]))[0])        # bf16(ln 3)
    G[0, 0] = ln3
    U[0, 0] = 2.0
    D[5, 0] = -0.5
    X = _bf16_experts(np.stack([G, U])[None], D[None])
    got = oracle.expert(X, 0, x.astype(np.float64), H, I)
    want = -0.5 * 2.0 * ln3 / (1 + 1 / np.exp(ln3))
    assert got[5] == pytest.approx(want, rel=1e-15)
    assert np.count_nonzero(got) == 1


# ----------------------------------------------------------------- layer
@pytest.mark.parametrize("fmt", ["nvfp4", "bf16"])
def test_sparse_equals_dense_masked(fmt):
    L = tiny_layer(fmt=fmt)
    x = testgen.make_x(11, 3, H)
    y, ids, w, gap = oracle.forward_layer(x, L)
    yd = oracle.forward_dense(x, L.router, L.routed, L.shared, K, I)
    np.testing.assert_array_equal(y, yd)


def test_identical_routed_experts_make_routing_irrelevant():
    """All routed experts equal -> y = f(x) + shared(x) whatever the routing,
    since the renormalised weights sum to 1."""
    L = tiny_layer(fmt="nvfp4")
    R = L.routed
    same = testgen.Experts("nvfp4", E, np.repeat(R.w13[:1], E, 0), np.repeat(R.w2[:1], E, 0),
                           np.repeat(R.w13_scale[:1], E, 0), np.repeat(R.w2_scale[:1], E, 0),
                           np.repeat(R.glob[:1], E, 0))
    x = testgen.make_x(4, 2, H)
    y, ids, w, _ = oracle.forward(x, L.router, same, L.shared, K, I)
    for t in range(2):
        xt = f64(x[t])
        want = oracle.expert(same, 0, xt, H, I) + oracle.expert(L.shared, 0, xt, H, I)
        np.testing.assert_allclose(y[t], want, rtol=1e-14, atol=1e-15)


def test_expert_relabelling_is_invisible():
    """Permuting router rows and routed experts together leaves y unchanged."""
    L = tiny_layer(fmt="nvfp4")
    perm = np.random.default_rng(5).permutation(E)
    R = L.routed
    P = testgen.Experts("nvfp4", E, R.w13[perm].copy(), R.w2[perm].copy(),
                        R.w13_scale[perm].copy(), R.w2_scale[perm].copy(), R.glob[perm].copy())
    x = testgen.make_x(8, 3, H)
    y, ids, _, _ = oracle.forward(x, L.router, L.routed, L.shared, K, I)
    y2, ids2, _, _ = oracle.forward(x, L.router[perm].copy(), P, L.shared, K, I)
    np.testing.assert_allclose(y2, y, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(perm[ids2], ids)


def test_tokens_are_independent():
    L = tiny_layer(fmt="nvfp4")
    x = testgen.make_x(9, 4, H)
    y, ids, w, gap = oracle.forward_layer(x, L)
    for t in range(4):
        y1, ids1, _, _ = oracle.forward_layer(x[t:t + 1], L)
        np.testing.assert_array_equal(y1[0], y[t])
        np.testing.assert_array_equal(ids1[0], ids[t])


def test_shared_expert_is_added_with_weight_one():
    L = tiny_layer(fmt="nvfp4")
    x = testgen.make_x(10, 2, H)
    y, _, _, _ = oracle.forward_layer(x, L)
    y0, _, _, _ = oracle.forward(x, L.router, L.routed, None, K, I)
    for t in range(2):
        sh = oracle.expert(L.shared, 0, f64(x[t]), H, I)
        np.testing.assert_allclose(y[t] - y0[t], sh, rtol=1e-12, atol=1e-14)


def test_forced_ids_reproduce_routing_when_equal():
    L = tiny_layer(fmt="nvfp4")
    x = testgen.make_x(12, 2, H)
    y, ids, w, _ = oracle.forward_layer(x, L)
    y2, ids2, w2, _ = oracle.forward_layer(x, L, forced_ids=ids[:, ::-1].copy())
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(np.sort(w2, 1), np.sort(w, 1))


def test_nvfp4_layer_equals_bf16_layer_on_grid_weights():
    """NVFP4 weights whose global is a power of two dequantise to bf16-exact
    values; a bf16 copy of those values (built from the OCP tables, not from
    the oracle's decoder) must give the identical layer output."""
    rng = np.random.default_rng(4)
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
    glob = 2.0 ** -10

    def rand_tensor(n, rows, cols):
        codes = rng.integers(0, 256, (n, rows, cols // 2), dtype=np.uint8)
        scales = rng.integers(0x28, 0x48, (n, rows, cols // 16), dtype=np.uint8)
        sval = np.array([2.0 ** (((b >> 3) & 15) - 7) * (1 + (b & 7) / 8) for b in range(256)])
        lo, hi = codes & 15, codes >> 4
        nib = np.stack([lo, hi], -1).reshape(n, rows, cols)
        vals = e2[nib] * np.repeat(sval[scales], 16, -1) * glob
        return codes, scales, vals

    c13, s13, v13 = rand_tensor(E + 1, 2 * I, H)
    c2, s2, v2 = rand_tensor(E + 1, H, I)
    g = np.full((E + 1, 3), glob, np.float32)

    def nv(sl):
        return testgen.Experts("nvfp4", len(range(*sl.indices(E + 1))),
                               c13[sl].reshape(-1, 2, I, H // 2).copy(), c2[sl].copy(),
                               s13[sl].reshape(-1, 2, I, H // 16).copy(), s2[sl].copy(),
                               g[sl].copy())

    def bf(sl):
        return _bf16_experts(v13[sl].reshape(-1, 2, I, H).astype(np.float32),
                             v2[sl].astype(np.float32))

    L = tiny_layer()
    x = testgen.make_x(13, 3, H)
    y_nv, ids_nv, _, _ = oracle.forward(x, L.router, nv(slice(0, E)), nv(slice(E, E + 1)), K, I)
    y_bf, ids_bf, _, _ = oracle.forward(x, L.router, bf(slice(0, E)), bf(slice(E, E + 1)), K, I)
    np.testing.assert_array_equal(ids_nv, ids_bf)
    np.testing.assert_array_equal(y_nv, y_bf)


# ----------------------------------------------------------------- dense NVFP4 GEMV
def _spec_decode(codes, scales, glob):
    """W [N, K] decoded in the test from the hand-written OCP tables (not the oracle)."""
    e2m1 = load_table("e2m1_values.txt")
    e4m3 = load_table("e4m3_values.txt")
    N, half = codes.shape
    K = half * 2
    W = np.empty((N, K), np.float64)
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            nib = (byte >> 4) if (k & 1) else (byte & 15)
            W[n, k] = e2m1[nib] * e4m3[int(scales[n, k // 16])] * glob
    return W


def _finite_scale_bytes(rng, shape):
    """Scale bytes drawn from the hand-written E4M3 table's finite entries."""
    table = load_table("e4m3_values.txt")
    ok = np.array(sorted(b for b, v in table.items() if v == v), np.uint8)
    return rng.choice(ok, size=shape).astype(np.uint8)


def test_gemv_one_hot_input_reads_one_decoded_column():
    """x = e_c gives y[n] = W[n][c] exactly, with W from the spec tables."""
    rng = np.random.default_rng(5)
    N, K = 11, 64
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = _finite_scale_bytes(rng, (N, K // 16))
    glob = 0.75
    W = _spec_decode(codes, scales, glob)
    for c in (0, 1, 17, 62, 63):
        x = np.zeros((1, K), np.uint16)
        x[0, c] = 0x3F80                                   # bf16 1.0
        y = oracle.gemv_nvfp4(x, codes, scales, glob)
        np.testing.assert_array_equal(y[0], W[:, c])


@pytest.mark.parametrize("N,K,B", [(7, 32, 1), (40, 96, 3), (5, 256, 8)])
def test_gemv_matches_spec_decode_times_numpy(N, K, B):
    """Against numpy's product of the spec-table decode (a non-square W catches a
    transposed operand, random bytes a wrong nibble or scale index)."""
    rng = np.random.default_rng(N * K + B)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = _finite_scale_bytes(rng, (N, K // 16))
    glob = 2.0 ** -7
    x = testgen.make_x(N + K, B, K)
    y = oracle.gemv_nvfp4(x, codes, scales, glob)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ _spec_decode(codes, scales, glob).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)


def test_gemv_is_linear_in_the_global_scale_and_rows_are_independent():
    c, s, g = testgen.make_dense(2, 0, 3, 24, 128)
    x = testgen.make_x(9, 2, 128)
    y = oracle.gemv_nvfp4(x, c, s, g)
    np.testing.assert_array_equal(oracle.gemv_nvfp4(x, c, s, 2.0 * g), 2.0 * y)
    perm = np.random.default_rng(1).permutation(24)
    np.testing.assert_array_equal(oracle.gemv_nvfp4(x, c[perm].copy(), s[perm].copy(), g), y[:, perm])


# ----------------------------------------------------------------- RMSNorm, residual
def _bf16(v: float) -> int:
    """bf16 bits of a value known to be exactly representable."""
    b = int(f32_to_bf16_bits_exact(np.array([v], np.float32))[0])
    assert float(f64(np.array([b], np.uint16))[0]) == v
    return b


def test_bf16_rounding_is_identity_on_every_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    vals = f64(bits[finite])
    assert np.array_equal(oracle.bf16_rne(vals), bits[finite])


def test_bf16_rounding_ties_go_to_even_and_off_ties_to_nearest():
    # 1 + 2^-8 lies halfway between 1 (mantissa 0, even) and 1 + 2^-7 (odd)
    assert oracle.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_rne(-(1.0 + 2.0 ** -8 - 2.0 ** -40)) == 0xBF80
    assert oracle.bf16_rne(-0.0) == 0x8000
    # the largest finite bf16 is (2 - 2^-7) 2^127; beyond the last tie -> inf
    assert oracle.bf16_rne((2 - 2.0 ** -7) * 2.0 ** 127) == 0x7F7F
    assert oracle.bf16_rne((2 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80
    # subnormal grid 2^-133: 1.5 steps rounds to 2 steps (even), 2.5 to 2
    assert oracle.bf16_rne(1.5 * 2.0 ** -133) == 0x0002
    assert oracle.bf16_rne(2.5 * 2.0 ** -133) == 0x0002
    assert oracle.bf16_rne(0.5 * 2.0 ** -133) == 0x0000


def test_rmsnorm_worked_example():
    # x = (3, 4): mean square 12.5, 1/sqrt(12.5) = 0.282842712...; so
    # xn = (0.848528..., 1.131370...), which lie in [0.5, 1) and [1, 2) with bf16
    # spacing 2^-8 and 2^-7: 217.2 and 144.8 steps -> 217 * 2^-8 and 145 * 2^-7.
    x = np.array([[_bf16(3.0), _bf16(4.0)]], np.uint16)
    w = np.array([_bf16(1.0), _bf16(1.0)], np.uint16)
    got = f64(oracle.rmsnorm_bf16(x, w, 0.0))[0]
    assert got.tolist() == [217 * 2.0 ** -8, 145 * 2.0 ** -7]


def test_rmsnorm_of_a_constant_row_is_the_weight():
    """mean of c^2 over the row is c^2: xn = sign(c) w exactly (eps = 0) for
    any c and any row length; a wrong mean (sum, or a dropped square) fails."""
    H = 48
    w = np.array([_bf16(v) for v in [0.5, -1.25, 3.0, 0.0] * (H // 4)], np.uint16)
    for c in [1.0, -2.0, 0.375, 40.0]:
        x = np.full((1, H), _bf16(c), np.uint16)
        got = f64(oracle.rmsnorm_bf16(x, w, 0.0))[0]
        assert np.array_equal(got, np.sign(c) * f64(w)), c


def test_rmsnorm_epsilon_sits_inside_the_root():
    # x = 1 everywhere: 1 / sqrt(1 + 3) = 1/2 exactly
    x = np.full((2, 16), _bf16(1.0), np.uint16)
    w = np.full(16, _bf16(1.0), np.uint16)
    assert np.all(f64(oracle.rmsnorm_bf16(x, w, 3.0)) == 0.5)
    # x = 0 with eps > 0 gives 0, not NaN
    z = np.zeros((1, 16), np.uint16)
    assert np.all(f64(oracle.rmsnorm_bf16(z, w, 1e-6)) == 0.0)


def test_rmsnorm_symmetries():
    x = testgen.make_x(9, 3, 256)
    w = testgen.make_x(10, 1, 256)[0]
    base = f64(oracle.rmsnorm_bf16(x, w, 0.0))
    # sign flip of x (bf16 sign bit) flips the output
    assert np.array_equal(f64(oracle.rmsnorm_bf16(x ^ np.uint16(0x8000), w, 0.0)), -base)
    # x scaled by a power of two (exponent field + 3) leaves it unchanged
    assert np.array_equal(f64(oracle.rmsnorm_bf16(x + np.uint16(3 << 7), w, 0.0)), base)
    # w scaled by 2 scales the output by 2 (the rounding commutes with it)
    assert np.array_equal(f64(oracle.rmsnorm_bf16(x, w + np.uint16(1 << 7), 0.0)), 2 * base)
    # rows are independent
    assert np.array_equal(f64(oracle.rmsnorm_bf16(x[1:2], w, 0.0)), base[1:2])


def test_fused_layer_reduces_to_the_plain_layer():
    """x with entries +-1 has mean square 1, so with w = 1 and eps = 0 the norm
    returns x itself and the fused layer is the plain one; a residual of zeros
    adds nothing; a residual r adds r exactly (to fp64 rounding)."""
    L = tiny_layer(seed=4)
    rng = np.random.default_rng(3)
    x = np.where(rng.random((3, H)) < 0.5, _bf16(1.0), _bf16(-1.0)).astype(np.uint16)
    ones = np.full(H, _bf16(1.0), np.uint16)
    y0, ids0, w0, _ = oracle.forward_layer(x, L)
    y1, ids1, w1, _, xn = oracle.forward_fused(x, L, norm_w=ones, eps=0.0,
                                               residual=np.zeros_like(x))
    assert np.array_equal(xn, x)
    assert np.array_equal(ids0, ids1) and np.array_equal(w0, w1)
    assert np.array_equal(y0, y1)
    r = testgen.make_x(12, 3, H)
    y2 = oracle.forward_fused(x, L, norm_w=ones, eps=0.0, residual=r)[0]
    assert np.allclose(y2 - y0, f64(r), rtol=0, atol=1e-12 * np.abs(y0).max())


def test_fused_layer_normalises_before_routing():
    """Scaling x by a power of two changes the plain layer but not the fused one."""
    L = tiny_layer(seed=6)
    x = testgen.make_x(13, 2, H)
    w = testgen.make_x(14, 1, H)[0]
    a = oracle.forward_fused(x, L, norm_w=w, eps=0.0)
    b = oracle.forward_fused(x + np.uint16(2 << 7), L, norm_w=w, eps=0.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(oracle.forward_layer(x, L)[0],
                              oracle.forward_layer(x + np.uint16(2 << 7), L)[0])


# ----------------------------------------------------------------- MXFP8, shared-expert count
def test_e8m0_spec_values():
    """OCP MX v1.0 E8M0: bias 127, 2^-127 .. 2^127, 0xFF is NaN."""
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(128) == 2.0 and oracle.e8m0(126) == 0.5
    assert oracle.e8m0(0) == 2.0 ** -127 and oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))


def _mx_tensor(rng, n, rows, cols):
    """Random MXFP8 bytes (finite E4M3 elements from the hand-written table,
    scales 2^-8 .. 2^-3) and their values decoded in the test."""
    e4 = load_table("e4m3_values.txt")
    ok = np.array(sorted(b for b, v in e4.items() if v == v), np.uint8)
    el = rng.choice(ok, size=(n, rows, cols)).astype(np.uint8)
    sc = rng.integers(119, 125, (n, rows, cols // 32), dtype=np.uint8)
    lut = np.array([e4.get(b, np.nan) for b in range(256)])
    vals = lut[el] * np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, -1)
    return el, sc, vals


def test_mxfp8_layer_equals_bf16_layer_on_grid_weights():
    """MXFP8 values (E4M3 element x power-of-two scale) are bf16-exact here; a
    bf16 copy built from the hand-written E4M3 table, not from the oracle's
    decoder, must give the identical layer (routed and 2 shared experts)."""
    rng = np.random.default_rng(8)
    HH, II = 64, 32
    e13, s13, v13 = _mx_tensor(rng, E + 2, 2 * II, HH)
    e2, s2, v2 = _mx_tensor(rng, E + 2, HH, II)

    def mx(sl):
        n = len(range(*sl.indices(E + 2)))
        return testgen.Experts("mxfp8", n, e13[sl].reshape(-1, 2, II, HH).copy(), e2[sl].copy(),
                               s13[sl].reshape(-1, 2, II, HH // 32).copy(), s2[sl].copy(), None)

    def bf(sl):
        return _bf16_experts(v13[sl].reshape(-1, 2, II, HH).astype(np.float32),
                             v2[sl].astype(np.float32))

    R = testgen.make_router(5, 0, E, HH, 0.5)
    x = testgen.make_x(14, 3, HH)
    y_mx, ids_mx, _, _ = oracle.forward(x, R, mx(slice(0, E)), mx(slice(E, E + 2)), K, II)
    y_bf, ids_bf, _, _ = oracle.forward(x, R, bf(slice(0, E)), bf(slice(E, E + 2)), K, II)
    np.testing.assert_array_equal(ids_mx, ids_bf)
    np.testing.assert_array_equal(y_mx, y_bf)


def test_mxfp8_packer_follows_the_mx_conversion_rule():
    """Per 32-block: scale 2^(floor(log2 amax) - 8); amax maps into [256, 512)
    (saturating to 448 above the last tie at 464); grid values come back exactly;
    an all-zero block is byte 0 with zero elements."""
    e4 = {b: oracle.e4m3(b) for b in range(256)}      # pinned against the spec table
    vals = np.zeros((3, 32), np.float32)
    vals[0] = 2.0 ** -4 * np.array([1, -1.5, 0.25, 3, 0.5, 1.75] * 5 + [0, 1], np.float32)
    vals[1, 0], vals[1, 1] = 1.9375, 1.0                     # amax 1.9375 -> 496 -> 448
    w = f32_to_bf16_bits_exact(vals)
    el, sc = testgen.quantize_mxfp8(w)
    # amax 3 * 2^-4 lies in [2^-3, 2^-2): exponent -3; amax 1.9375 in [1, 2): exponent 0
    assert sc[0, 0] == 127 + (-3 - 8) and sc[1, 0] == 127 + (0 - 8) and sc[2, 0] == 0
    dec = np.array([[e4[int(b)] for b in row] for row in el]) * \
        np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, -1)
    dec[2] = 0.0
    np.testing.assert_array_equal(dec[0], vals[0])
    assert dec[1, 0] == 448 * 2.0 ** -8 and dec[1, 1] == 1.0
    assert not el[2].any()


def test_mxfp8_round_trip_error_is_within_half_an_e4m3_step():
    w = testgen.make_x(15, 64, 256)
    el, sc = testgen.quantize_mxfp8(w)
    lut = np.array([oracle.e4m3(b) for b in range(256)])
    dec = lut[el] * np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, -1)
    v = f64(w)
    # half the relative step 2^-3 of a normal E4M3 value; subnormals have step
    # 2^-9 * scale; values above 448 * scale (only the top of [256, 512) that
    # the block maximum maps into) saturate to 448 * scale
    scale = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, -1)
    sat = np.abs(v) > 448 * scale
    bound = np.where(sat, np.abs(v) - 448 * scale,
                     np.maximum(np.abs(v) * 2.0 ** -4, scale * 2.0 ** -10))
    assert np.all(np.abs(dec - v) <= bound)
    assert np.all(np.abs(v) / scale < 512)


def test_every_shared_expert_is_added_with_weight_one():
    L = testgen.make_layer(3, 0, "nvfp4", H, I, E, K, 0.5, n_shared=2)
    x = testgen.make_x(16, 2, H)
    y, ids, _, _ = oracle.forward_layer(x, L)
    y0, ids0, _, _ = oracle.forward(x, L.router, L.routed, None, K, I)
    np.testing.assert_array_equal(ids, ids0)
    for t in range(2):
        d = oracle.expert(L.shared, 0, f64(x[t]), H, I) + oracle.expert(L.shared, 1, f64(x[t]), H, I)
        np.testing.assert_allclose(y[t] - y0[t], d, rtol=1e-12, atol=1e-14)
    # two identical shared experts count twice
    L1 = testgen.make_layer(3, 0, "nvfp4", H, I, E, K, 0.5, n_shared=1)
    sh2 = testgen.Experts("nvfp4", 2, np.concatenate([L1.shared.w13] * 2),
                          np.concatenate([L1.shared.w2] * 2),
                          np.concatenate([L1.shared.w13_scale] * 2),
                          np.concatenate([L1.shared.w2_scale] * 2),
                          np.concatenate([L1.shared.glob] * 2))
    y1 = oracle.forward(x, L1.router, L1.routed, L1.shared, K, I)[0]
    y2 = oracle.forward(x, L1.router, L1.routed, sh2, K, I)[0]
    np.testing.assert_allclose(y2 - y0, 2 * (y1 - y0), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- Four Over Six (W4A4)
G0 = 2.0 ** -10          # global of a vector whose maximum is 2688 * 2^-10 = 2.625
E2 = np.array([6, 4, 3, 2, 1.5, 1, .5, 0, -6, -4, -3, -2, -1.5, -1, -.5, 0.0])


def _vec(*blocks):
    """A vector fixing the global at 2^-10 (first block holds 2.625) followed by the blocks."""
    first = np.zeros(16)
    first[0] = 2688 * G0
    return np.concatenate([first, *blocks]).astype(np.float32)


def test_fp4_46_exact_block_keeps_the_max_to_6_scale():
    blk = E2 * 16 * G0                               # scale 16 = 2^4: E4M3 byte 0x58
    codes, scales, g, vals = oracle.quant_fp4_46(_vec(blk))
    assert g == G0
    assert scales.tolist() == [0x7E, 0x58]          # 448 for 2.625 = 6 * 448 * 2^-10
    np.testing.assert_array_equal(vals, _vec(blk).astype(np.float64))


def test_fp4_46_takes_max_to_4_when_it_reconstructs_better():
    blk = np.array([4, 3, 2, 1.5, 1, .5, 0, -4, -3, -2, -1.5, -1, -.5, 0, 2, 1]) * 16 * G0
    # max -> 6 needs scale 10.67 (E4M3 rounds it to 11: 64/11 is not on the grid);
    # max -> 4 needs exactly 16
    codes, scales, g, vals = oracle.quant_fp4_46(_vec(blk))
    assert scales[1] == 0x58
    np.testing.assert_array_equal(vals[16:], blk)


def test_fp4_46_tie_keeps_the_max_to_6_scale():
    blk = np.full(16, 96 * G0)                       # 6 * 16 g and 4 * 24 g: both exact
    _, scales, _, vals = oracle.quant_fp4_46(_vec(blk))
    assert scales[1] == 0x58                         # 16, not 24 (0x5C)
    np.testing.assert_array_equal(vals[16:], blk)


def test_fp4_46_zero_and_power_of_two_scaling():
    c, s, g, v = oracle.quant_fp4_46(np.zeros(32, np.float32))
    assert g == 0.0 and not s.any() and not v.any()
    x = f64(testgen.make_x(30, 1, 256)[0]).astype(np.float32)
    c1, s1, g1, v1 = oracle.quant_fp4_46(x)
    c2, s2, g2, v2 = oracle.quant_fp4_46(x * np.float32(8))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert g2 == 8 * g1 and np.array_equal(v2, 8 * v1)


def test_fp4_46_departs_from_the_max_to_6_packer_only_to_reconstruct_better():
    """The input generator's NVFP4 packer is the max->6 rule with the same
    global (amax / 2688); the oracle's choice equals it block by block, or has
    a smaller MAE (and does somewhere)."""
    w = testgen.make_x(31, 1, 4096)
    c6p, s6, g6 = testgen.quantize_nvfp4(w)
    c6 = np.stack([c6p[0] & 15, c6p[0] >> 4], -1).reshape(-1)
    v = f64(w[0])
    codes, scales, g, vals = oracle.quant_fp4_46(v.astype(np.float32))
    assert np.float32(g) == np.float32(g6)
    e2 = np.array([oracle.e2m1(i) for i in range(16)])
    e4 = np.array([oracle.e4m3(b) for b in range(256)])
    v6 = e2[c6] * np.repeat(e4[s6[0]], 16) * g6
    n_four = 0
    for b in range(v.size // 16):
        sl = slice(16 * b, 16 * b + 16)
        if scales[b] == s6[0, b] and np.array_equal(codes[sl], c6[sl]):
            continue
        n_four += 1
        assert np.abs(vals[sl] - v[sl]).sum() < np.abs(v6[sl] - v[sl]).sum() * (1 + 1e-6)
    assert 0 < n_four < v.size // 16


def test_w4a4_layer_override_and_token_independence():
    L = tiny_layer(seed=7)
    x = testgen.make_x(32, 3, H)
    y, ids, w, gap, h = oracle.forward_w4a4(x, L)
    y2, ids2, _, _, h2 = oracle.forward_w4a4(x, L, h_in=h)
    assert np.array_equal(y, y2) and np.array_equal(h, h2)
    y1, ids1, _, _, h1 = oracle.forward_w4a4(x[1:2].copy(), L)
    assert np.array_equal(y1[0], y[1]) and np.array_equal(h1[0], h[1])
    # the routing is the plain layer's (the router stays in high precision)
    assert np.array_equal(ids, oracle.forward_layer(x, L)[1])
    # an h overridden with zeros leaves no expert output
    y0 = oracle.forward_w4a4(x, L, h_in=np.zeros_like(h))[0]
    assert not y0.any()


# ------------------------------------------------------- W4A4 layer composition
# Pins of or_forward_w4a4 against numpy products of weights decoded from the
# hand-written OCP tables: special cases where the activation quantiser is
# exact reduce the W4A4 layer to the W4A16 one, and the quantiser (pinned
# above) is otherwise used only as a step.  A slip in the composition (gate
# and up fed the unquantised x, the shared expert fed x instead of its
# quantisation, h quantised without its bf16 rounding, a routing weight
# dropped or a slot out of order) fails one of them.
HW, IW = 64, 32
E4M3_EXACT = [0.25, 0.5, 1.0, 1.5, 2.0, 3.0, 8.0, 14.0, 40.0, 96.0]   # below 448, exact in E4M3
GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])


def _exact_fp4_vector(rng, n):
    """A vector the Four-Over-Six quantiser reproduces exactly: amax = 21 * 2^m
    makes the global amax / 2688 = 2^(m - 7) a power of two, block 0 holds
    that maximum (E4M3 scale 448), every block is E2M1 values times an E4M3
    value times the global, with its maximum coded +-6 (scale exact, MAE 0,
    which the max->4 candidate cannot beat).  Every element has at most six
    significant bits, so it is exact in bf16."""
    g = 2.0 ** (int(rng.integers(-3, 3)) - 7)
    v = np.empty(n)
    for b in range(n // 16):
        S = 448.0 if b == 0 else float(rng.choice(E4M3_EXACT))
        blk = rng.choice(GRID, 16) * rng.choice([-1.0, 1.0], 16)
        blk[rng.integers(16)] = 6.0 * rng.choice([-1.0, 1.0])
        v[16 * b:16 * b + 16] = blk * S * g
    return v


def _bf16_rne_np(v):
    """fp64 -> nearest bf16 value, ties to even (numpy): 8 significant bits,
    spacing 2^(e - 8) for v = m 2^e (m in [0.5, 1)); below the smallest
    normal 2^-126 the spacing stays 2^-133 (subnormals, flushing to 0)."""
    v = np.asarray(v, np.float64)
    e = np.maximum(np.frexp(v)[1], -125)
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)


def _e4m3_closed_form(b: int) -> float:
    """OCP E4M3FN: sign bit 7, exponent bits 6-3 (bias 7), mantissa bits 2-0;
    exponent 0 is subnormal (m / 8 * 2^-6); S.1111.111 is NaN."""
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_e4m3_closed_form_agrees_with_the_hand_written_table():
    for b, v in load_table("e4m3_values.txt").items():
        c = _e4m3_closed_form(b)
        assert (math.isnan(v) and math.isnan(c)) or c == v, hex(b)


def _decode_full(codes, scales, glob):
    """W [N, K] from the hand-written E2M1 table and the E4M3 closed form."""
    e2m1 = load_table("e2m1_values.txt")
    t2 = np.array([e2m1[i] for i in range(16)])
    t4 = np.array([_e4m3_closed_form(b) for b in range(256)])
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1)
    return t2[nib] * np.repeat(t4[scales], 16, axis=1) * glob


def _mats(X, e):
    """Gate, up, down of expert e of a host NVFP4 set, decoded in the test."""
    return (_decode_full(X.w13[e, 0], X.w13_scale[e, 0], float(X.glob[e, 0])),
            _decode_full(X.w13[e, 1], X.w13_scale[e, 1], float(X.glob[e, 1])),
            _decode_full(X.w2[e], X.w2_scale[e], float(X.glob[e, 2])))


def _slots(L, ids_t):
    """(expert set, index) of each h slot: routed ids ascending, then shared."""
    return [(L.routed, int(e)) for e in sorted(ids_t.tolist())] + [(L.shared, 0)]


def _silu_mul(g, u):
    return g / (1.0 + np.exp(-g)) * u


def test_w4a4_h_equals_the_w4a16_h_when_x_is_on_the_fp4_grid():
    L = tiny_layer(seed=11, H=HW, I=IW)
    rng = np.random.default_rng(5)
    xv = np.stack([_exact_fp4_vector(rng, HW) for _ in range(3)])
    for t in range(3):                               # the quantiser reproduces x
        np.testing.assert_array_equal(oracle.quant_fp4_46(xv[t].astype(np.float32))[3], xv[t])
    x = f32_to_bf16_bits_exact(xv.astype(np.float32))
    y, ids, w, gap, h = oracle.forward_w4a4(x, L)
    assert np.array_equal(ids, oracle.forward_layer(x, L)[1])
    for t in range(3):
        for s, (X, e) in enumerate(_slots(L, ids[t])):
            G, U, _ = _mats(X, e)
            want = _bf16_rne_np(_silu_mul(G @ xv[t], U @ xv[t]))
            np.testing.assert_array_equal(f64(h[t, s]), want)


def test_w4a4_down_and_combine_reduce_to_numpy_when_h_is_on_the_fp4_grid():
    L = tiny_layer(seed=12, H=HW, I=IW)
    x = testgen.make_x(33, 3, HW)
    rng = np.random.default_rng(6)
    hv = np.stack([np.stack([_exact_fp4_vector(rng, IW) for _ in range(L.K + 1)])
                   for _ in range(3)])
    y, ids, w, gap, _ = oracle.forward_w4a4(x, L, h_in=f32_to_bf16_bits_exact(
        hv.astype(np.float32)))
    ids_p, w_p, _, _ = oracle.route(x, L.router, L.K)      # the plain layer's routing
    np.testing.assert_array_equal(ids, ids_p)
    for t in range(3):
        wt = dict(zip(ids[t].tolist(), w[t].tolist()))
        want = np.zeros(HW)
        for s, (X, e) in enumerate(_slots(L, ids[t])):
            D = _mats(X, e)[2]
            want += (wt[e] if X is L.routed else 1.0) * (D @ hv[t, s])
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sum(wt.values()), 1.0, rtol=1e-12)


def test_w4a4_experts_read_the_quantised_x_and_the_bf16_h():
    """General x: gate and up of every slot (the shared one too) read the
    quantiser's x, h is SiLU(g) * u rounded to bf16, and the down GEMV reads
    the quantiser's image of that bf16 h."""
    L = tiny_layer(seed=13, H=HW, I=IW)
    x = testgen.make_x(34, 2, HW)
    y, ids, w, gap, h = oracle.forward_w4a4(x, L)
    for t in range(2):
        xq = oracle.quant_fp4_46(f64(x[t]).astype(np.float32))[3]
        assert not np.array_equal(xq, f64(x[t]))     # the quantisation changes this x
        wt = dict(zip(ids[t].tolist(), w[t].tolist()))
        want = np.zeros(HW)
        for s, (X, e) in enumerate(_slots(L, ids[t])):
            G, U, D = _mats(X, e)
            hb = _bf16_rne_np(_silu_mul(G @ xq, U @ xq))
            np.testing.assert_array_equal(f64(h[t, s]), hb)
            hq = oracle.quant_fp4_46(hb.astype(np.float32))[3]
            want += (wt[e] if X is L.routed else 1.0) * (D @ hq)
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-14)
