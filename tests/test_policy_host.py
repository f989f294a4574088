"""The library's host-side loop policy against the oracle's, case by case (plain integer and
comparison logic, so equal results): block lengths from draft uncertainties and draft read
positions after a round, on seeded random drafts, plus the host validation."""
import numpy as np
import pytest

import gqa_decode_attention_amd as ga
import oracle


def _lib():
    import os
    if not os.path.exists(ga.LIB_PATH):
        from gqa_decode_attention_amd.build import build
        build()
    return ga.load()


def test_block_length_equals_the_oracle():
    _lib()
    g = np.random.default_rng(70)
    for _ in range(2000):
        n = int(g.integers(0, 40))
        u = g.exponential(0.6, n).astype(np.float32).tolist()
        tau = float(np.float32(g.choice([0.5, 1.0, 2.0, 4.0])))
        k_min = int(g.integers(1, 9))
        k_max = int(g.integers(k_min, 33))
        assert ga.next_block_len(u, tau, k_min, k_max) == oracle.next_block_len(u, tau, k_min, k_max)


def test_recycle_position_equals_the_oracle():
    _lib()
    g = np.random.default_rng(71)
    for _ in range(4000):
        n = int(g.integers(1, 30))
        d = g.integers(0, 6, n).tolist()            # a small alphabet: matches are frequent
        pos = int(g.integers(0, n + 3))
        k = int(g.integers(1, 17))
        a = int(g.integers(0, k + 1))
        corr = None if a == k else int(g.integers(0, 6))
        w = int(g.integers(0, 6))
        assert ga.recycle_draft(d, pos, k, a, corr, w) == oracle.recycle_draft(d, pos, k, a, corr, w)


def test_policy_validation():
    lib = _lib()
    with pytest.raises(ga.AsrError):
        ga.next_block_len([0.1], 1.0, 0, 4)
    with pytest.raises(ga.AsrError):
        ga.next_block_len([0.1], 1.0, 5, 4)
    with pytest.raises(ga.AsrError):
        ga.next_block_len([0.1], 1.0, 1, 33)
    with pytest.raises(ga.AsrError):
        ga.recycle_draft([1, 2], 0, 2, 3, 5, 1)     # more accepted than verified
    with pytest.raises(ga.AsrError):
        ga.recycle_draft([1, 2], -1, 2, 0, 5, 1)
    with pytest.raises(ga.AsrError):
        ga.recycle_draft([1, 2], 0, 2, 0, 5, -1)
    assert lib.asr_next_block_len(None, 0, 1.0, 4, 8) == 1
    assert lib.asr_next_block_len(None, 2, 1.0, 4, 8) == -1
    assert lib.asr_recycle_draft(None, 0, 3, 2, 1, 7, 4) == 5


def test_mixed_acceptance_validates_on_the_host():
    import ctypes
    lib = _lib()
    fake = ctypes.c_void_p(0x1000)
    nb = (ctypes.c_int32 * 3)(2, 0, 4)
    call = lambda B, sizes: lib.asr_accept_greedy_mixed(fake, fake, B, sizes, None, fake, 64, fake, fake, fake, None)
    assert call(0, None) == 0
    assert call(3, ctypes.cast(nb, ctypes.c_void_p)) == -1        # a block of size 0
    assert call(2, None) == -1
    big = (ctypes.c_int32 * 65)(*([1] * 65))
    assert call(65, ctypes.cast(big, ctypes.c_void_p)) == -1
