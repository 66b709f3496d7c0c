"""The seeded input generator: determinism, shapes, distributions, bf16 rounding."""
import numpy as np

import kda_inputs as ki


def test_same_seed_same_bytes():
    a = ki.token_inputs(7, 33, 2)
    b = ki.token_inputs(7, 33, 2)
    for x, y in zip((a.q, a.k, a.v, a.z, a.b, a.g), (b.q, b.k, b.v, b.z, b.b, b.g)):
        np.testing.assert_array_equal(x, y)
    c = ki.token_inputs(8, 33, 2)
    assert not np.array_equal(a.q, c.q)


def test_row_prefix_is_stable():
    # drawing more rows does not change the first ones (decode steps and samples rely on it)
    np.testing.assert_array_equal(ki.normal(3, 10, (300000, 4), 1.0)[:200000], ki.normal(3, 10, (200000, 4), 1.0))


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38, 1e-40, 0.0], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 1.5*2^-8 rounds up
    got = ki.bf16_bits_to_f32(ki.to_bf16_bits(x))
    np.testing.assert_array_equal(got[:4], np.array([1.0, 1.0, 1.0078125, -2.5], np.float32))
    assert got[6] == 0.0
    y = np.random.default_rng(0).normal(size=10000).astype(np.float32)
    r = ki.bf16_bits_to_f32(ki.to_bf16_bits(y))
    assert np.max(np.abs(r - y) / np.abs(y)) <= 2.0 ** -8  # bf16: 8 significant bits


def test_case_shapes_and_distributions():
    c0 = ki.case0_decode()
    assert c0.state.shape == (1, 4, 128, 128) and not c0.state.any()
    s = c0.step(5)
    assert s.q.shape == (1, 512) and s.b.shape == (1, 4)
    p = c0.params
    assert p.conv_w.shape == (1536, 4) and p.dt_bias.shape == (512,) and p.A_log.shape == (4,)
    assert p.dt_bias.min() >= -1 and p.dt_bias.max() < 1 and p.A_log.min() >= -2 and p.A_log.max() < 1
    assert abs(np.std(p.conv_w) - 0.5) < 0.03
    pf = ki.case0_prefill()
    assert pf.x.q.dtype == np.uint16 and pf.N == 64
    # the prefill case is the bf16 rounding of the decode case's tokens
    np.testing.assert_array_equal(ki.bf16_bits_to_f32(pf.x.q[5:6]), ki.bf16_bits_to_f32(ki.to_bf16_bits(s.q)))
    lens = ki.case3_lengths()
    assert len(lens) == 16 and lens.min() >= 512 and lens.max() <= 4096
