"""The seeded input generator: stream definition, distributions, determinism."""
import numpy as np

import testgen
from tests.helpers import GOLDEN, bf16_bits_to_f32


def test_splitmix64_known_answers():
    for line in (GOLDEN / "splitmix64_vectors.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if line:
            n, v = line.split()
            assert testgen.splitmix_at(0, int(n)) == int(v, 16)


def test_streams_are_deterministic_and_distinct():
    a = testgen.normal_bf16(1, 0, 3, 1, 0.02, 4096)
    b = testgen.normal_bf16(1, 0, 3, 1, 0.02, 4096)
    np.testing.assert_array_equal(a, b)
    for key in [(2, 0, 3, 1), (1, 1, 3, 1), (1, 0, 4, 1), (1, 0, 3, 2)]:
        c = testgen.normal_bf16(*key, 0.02, 4096)
        assert np.mean(a == c) < 0.1


def test_normal_moments():
    z = testgen.normal_f32(1, 0, 0, 4, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.std() - 1.0) < 5e-3
    # Irwin-Hall(12): excess kurtosis -0.1, bounded support +-6
    k = ((z - z.mean()) ** 4).mean() / z.var() ** 2 - 3
    assert -0.14 < k < -0.06
    assert np.abs(z).max() < 6.0


def test_weights_have_the_configured_sigma():
    w = bf16_bits_to_f32(testgen.normal_bf16(1, 0, 0, 1, 0.02, 1 << 20)).astype(np.float64)
    assert abs(w.std() - 0.02) < 2e-4


def test_bf16_round_to_nearest_even():
    f = np.float32
    cases = {1.0: 0x3F80, 1.00390625: 0x3F80, 1.01171875: 0x3F82, 1.0078125: 0x3F81,
             -2.0: 0xC000, 0.0: 0, 3.3895313892515355e38: 0x7F7F}
    for v, bits in cases.items():
        assert testgen.bf16_rne(float(f(v))) == bits, v


def test_x_layout_is_token_major():
    x = testgen.make_x(3, 4, 64)
    flat = testgen.normal_bf16(3, 0, 0, 4, 1.0, 4 * 64)
    np.testing.assert_array_equal(x.ravel(), flat)


def test_expert_streams_match_standalone_tensors():
    L = testgen.make_layer(2, 1, "bf16", 32, 16, 4, 2, 0.5)
    g = testgen.normal_bf16(2, 1, 3, 1, 0.5, 16 * 32).reshape(16, 32)
    np.testing.assert_array_equal(L.routed.w13[3, 0], g)
    d = testgen.normal_bf16(2, 1, 4, 3, 0.5, 32 * 16).reshape(32, 16)
    np.testing.assert_array_equal(L.shared.w2[0], d)
