"""Pins of the oracle's verify loop: the acceptance rule, the lm_head argmax, and the greedy
exactness of speculative rounds ("Can CTC make Qwen3-ASR faster?", section 03 "Greedy
exactness"; section 11 Phase A steps 3-5: the one-token shift, an oracle draft, mismatches
injected at controlled positions)."""
import math

import numpy as np
import pytest

from oracle import (F16, BlockConfig, HeadConfig, KVCache, LayerWeights, MlpConfig, MlpWeights, TinyModel,
                    accept_greedy, argmax_first, embed, greedy_decode, kv_append, lm_head_logits,
                    speculative_round, widen)


def test_accept_greedy_cases():
    assert accept_greedy([5, 6, 7], [5, 6, 7]) == (3, None, 3)        # all accepted
    assert accept_greedy([5, 6, 7], [9, 6, 7]) == (0, 9, 1)           # first candidate wrong
    assert accept_greedy([5, 6, 7], [5, 1, 7]) == (1, 1, 2)           # mismatch in the middle
    assert accept_greedy([5, 6, 7], [5, 6, 2]) == (2, 2, 3)           # last candidate wrong
    assert accept_greedy([4], [4]) == (1, None, 1)


def test_argmax_ties_go_to_the_smallest_id():
    logits = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0], [-1.0, -2.0, -1.0, -5.0]])
    assert argmax_first(logits).tolist() == [1, 0, 0]


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def test_lm_head_matches_brute_force():
    H, V = 12, 30
    g = np.random.default_rng(1)
    gain = widen(_f16(1 + 0.02 * g.standard_normal(H)), F16)
    w = widen(_f16(0.3 * g.standard_normal((V, H))), F16)
    h = g.standard_normal((2, H))
    lg = lm_head_logits(HeadConfig(hidden=H, vocab=V), gain, w, h)
    for r in range(2):
        ms = math.fsum(v * v for v in h[r]) / H
        y = [h[r, i] * gain[i] / math.sqrt(ms + 1e-6) for i in range(H)]
        want = [math.fsum(w[t, i] * y[i] for i in range(H)) for t in range(V)]
        assert np.max(np.abs(lg[r] - want)) < 1e-12 * np.max(np.abs(want))
        assert argmax_first(lg[r:r + 1])[0] == int(np.argmax(want))


def _model(seed, n_layers=2, V=50):
    acfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    mcfg = MlpConfig(hidden=32, intermediate=48)
    hcfg = HeadConfig(hidden=32, vocab=V)
    g = np.random.default_rng(seed)
    layers = []
    for _ in range(n_layers):
        nqkv = (4 + 2 * 2) * 16
        aw = dict(input_norm_w=_f16(1 + 0.02 * g.standard_normal(32)), w_qkv=_f16(0.3 * g.standard_normal((nqkv, 32))),
                  q_norm_w=_f16(1 + 0.02 * g.standard_normal(16)), k_norm_w=_f16(1 + 0.02 * g.standard_normal(16)),
                  w_o=_f16(0.1 * g.standard_normal((32, 64))))
        mw = dict(post_norm_w=_f16(1 + 0.02 * g.standard_normal(32)), w_gate=_f16(0.3 * g.standard_normal((48, 32))),
                  w_up=_f16(0.3 * g.standard_normal((48, 32))), w_down=_f16(0.1 * g.standard_normal((32, 48))))
        layers.append((LayerWeights.from_bits(aw, F16), MlpWeights.from_bits(mw, F16)))
    model = TinyModel(acfg, mcfg, hcfg, _f16(g.standard_normal((V, 32))), layers,
                      widen(_f16(1 + 0.02 * g.standard_normal(32)), F16), widen(_f16(0.5 * g.standard_normal((V, 32))), F16))
    caches = []
    for _ in range(n_layers):   # a prompt of 7 positions already in every layer's cache
        c = KVCache.empty(1, 2, 64, 16, F16)
        kv_append(c, _f16(g.standard_normal((1, 7, 2, 16))), _f16(g.standard_normal((1, 7, 2, 16))))
        caches.append(c)
    return model, caches


def test_embedding_is_a_row_lookup():
    model, _ = _model(3)
    assert np.array_equal(embed(model.embed_bits, [4, 0, 4]), model.embed_bits[[4, 0, 4]])


@pytest.mark.parametrize("k", [2, 4, 5])
def test_speculative_rounds_with_an_oracle_draft_commit_the_greedy_transcript(k):
    model, caches = _model(10)
    ref = [c.copy() for c in caches]
    want = greedy_decode(model, ref, 3, 12)
    got, last, accepted = [], 3, []
    while len(got) < 12:
        draft = (want[len(got):] + [0] * k)[:k]                # the transcript itself as the draft
        committed, a = speculative_round(model, caches, last, draft)
        got += committed
        accepted.append(a)
        last = got[-1]
    assert got[:12] == want
    assert all(a == k for a in accepted[:-1])                  # every round accepts the whole draft
    assert caches[0].lens[0] == 7 + len(got)                   # every committed token but the last is cached


@pytest.mark.parametrize("bad", [0, 1, 3])
def test_injected_mismatches_still_commit_the_greedy_transcript(bad):
    """A draft wrong at position `bad` of every round: the round commits the accepted prefix and
    the target's correction, crops the rejected rows, and the transcript is still greedy's."""
    k = 4
    model, caches = _model(11)
    ref = [c.copy() for c in caches]
    want = greedy_decode(model, ref, 5, 14)
    got, last = [], 5
    while len(got) < 14:
        draft = (want[len(got):] + [0] * k)[:k]
        draft[bad] = (draft[bad] + 1) % model.hcfg.vocab
        committed, a = speculative_round(model, caches, last, draft)
        assert a <= bad
        got += committed
        last = got[-1]
    assert got[:14] == want
    # every position both caches hold has the same K/V (the block path and the one-token path
    # store the same 16-bit values), and the cache holds every committed token but the last
    assert all(int(c.lens[0]) == 7 + len(got) for c in caches)
    for c, r in zip(caches, ref):
        n = min(int(c.lens[0]), int(r.lens[0]))
        assert np.array_equal(c.k[0, :, :n], r.k[0, :, :n]) and np.array_equal(c.v[0, :, :n], r.v[0, :, :n])
