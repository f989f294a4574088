"""The seeded input module: determinism, shapes, distributions, 16-bit rounding."""
import numpy as np

from oracle import BF16, F16, rne16, widen
from synth import inputs as si


def test_streams_are_deterministic_and_independent():
    a = si.normal_bits(4, 3, si.T_WQKV, 0, (8, 8), dtype=BF16)
    b = si.normal_bits(4, 3, si.T_WQKV, 0, (8, 8), dtype=BF16)
    c = si.normal_bits(4, 4, si.T_WQKV, 0, (8, 8), dtype=BF16)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_rounding_of_draws_is_nearest_even():
    # the generator's own converters agree with the oracle's table-based rounding
    g = np.random.default_rng(3)
    a = np.concatenate([g.standard_normal(100_000) * s for s in (1e-40, 1e-3, 0.02, 1.0, 1e3)])
    assert np.array_equal(si.to_bits(a, BF16), rne16(a, BF16))
    a16 = a[np.abs(a) < 6e4]
    assert np.array_equal(si.to_bits(a16, F16), rne16(a16, F16))


def test_weight_and_cache_distributions():
    w = si.layer_weights(1, 0, 1024, F16)
    assert w["w_qkv"].shape == (4096, 1024) and w["w_o"].shape == (1024, 2048)
    wq = widen(w["w_qkv"], F16)
    assert abs(wq.std() - 0.02) < 2e-4 and abs(wq.mean()) < 2e-4
    gi = widen(w["input_norm_w"], F16)
    assert abs(gi.mean() - 1) < 5e-3 and abs(gi.std() - 0.02) < 3e-3
    k, v = si.kv_rows(1, 0, 0, 64, F16)
    assert k.shape == (8, 64, 128) and abs(widen(k, F16).std() - 1) < 0.02


def test_lengths_and_choices():
    lens = si.kv_lengths(4, 64, 200, 1500)
    assert lens.shape == (64,) and lens.min() >= 200 and lens.max() <= 1500
    assert np.array_equal(lens, si.kv_lengths(4, 64, 200, 1500))
    ch = si.verify_choice(5, 64, 8)
    assert len(set(ch.tolist())) == 8 and ch.max() < 64
    assert all(0 <= si.accepted_prefix(3, k, i) <= k for k in (4, 8, 16) for i in range(20))
