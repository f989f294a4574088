"""Pins of the oracle's MLP and whole-decoder-layer composition: SiLU closed forms, brute force
with scalar loops, the residual and zero-weight cases, RMSNorm scale invariance, and the
layer = attention block (residual x) followed by the MLP."""
import math

import numpy as np
import pytest

from oracle import (F16, BlockConfig, KVCache, LayerWeights, MlpConfig, MlpWeights, decode, decoder_layer_decode,
                    decoder_layer_verify, mlp, silu, widen)


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def _mlp_weights(seed, H, I, zero_down=False, zero_up=False):
    g = np.random.default_rng(seed)
    bits = dict(post_norm_w=_f16(1 + 0.02 * g.standard_normal(H)), w_gate=_f16(0.3 * g.standard_normal((I, H))),
                w_up=_f16(0.3 * g.standard_normal((I, H))), w_down=_f16(0.3 * g.standard_normal((H, I))))
    if zero_down:
        bits["w_down"][:] = 0
    if zero_up:
        bits["w_up"][:] = 0
    return MlpWeights.from_bits(bits, F16)


def test_silu_closed_forms():
    assert silu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-30, 30, 601)
    # silu(x) - silu(-x) = x, and silu(x) = x * sigmoid(x)
    assert np.allclose(silu(x) - silu(-x), x, atol=1e-12)
    assert np.allclose(silu(x), x * (0.5 + 0.5 * np.tanh(x / 2)), atol=1e-12)
    assert abs(silu(np.array([40.0]))[0] - 40.0) < 1e-12 and abs(silu(np.array([-40.0]))[0]) < 1e-15


def test_mlp_matches_brute_force():
    H, I = 12, 20
    cfg = MlpConfig(hidden=H, intermediate=I)
    w = _mlp_weights(1, H, I)
    h = np.random.default_rng(2).standard_normal((3, H))
    out = mlp(cfg, w, h)
    for r in range(3):
        ms = math.fsum(v * v for v in h[r]) / H
        y = [h[r, i] * w.post_norm_w[i] / math.sqrt(ms + cfg.rms_eps) for i in range(H)]
        gate = [math.fsum(w.w_gate[f, i] * y[i] for i in range(H)) for f in range(I)]
        up = [math.fsum(w.w_up[f, i] * y[i] for i in range(H)) for f in range(I)]
        act = [gate[f] / (1 + math.exp(-gate[f])) * up[f] for f in range(I)]
        want = [h[r, o] + math.fsum(w.w_down[o, f] * act[f] for f in range(I)) for o in range(H)]
        assert np.max(np.abs(out[r] - want)) < 1e-12 * np.max(np.abs(want))


def test_zero_down_or_up_passes_the_residual_through():
    H, I = 16, 24
    cfg = MlpConfig(hidden=H, intermediate=I)
    h = np.random.default_rng(3).standard_normal((2, H))
    assert np.array_equal(mlp(cfg, _mlp_weights(4, H, I, zero_down=True), h), h)
    assert np.array_equal(mlp(cfg, _mlp_weights(4, H, I, zero_up=True), h), h)


def test_norm_makes_the_mlp_branch_scale_invariant():
    H, I = 16, 24
    cfg = MlpConfig(hidden=H, intermediate=I, rms_eps=0.0)
    w = _mlp_weights(5, H, I)
    h = np.random.default_rng(6).standard_normal((2, H))
    assert np.allclose(mlp(cfg, w, 7.0 * h) - 7.0 * h, mlp(cfg, w, h) - h, rtol=1e-12, atol=1e-12)


def _attn(seed, cfg, lens, capacity):
    g = np.random.default_rng(seed)
    nqkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    wb = dict(input_norm_w=_f16(1 + 0.02 * g.standard_normal(cfg.hidden)),
              w_qkv=_f16(0.3 * g.standard_normal((nqkv, cfg.hidden))),
              q_norm_w=_f16(1 + 0.02 * g.standard_normal(cfg.head_dim)),
              k_norm_w=_f16(1 + 0.02 * g.standard_normal(cfg.head_dim)),
              w_o=_f16(0.3 * g.standard_normal((cfg.hidden, cfg.n_q_heads * cfg.head_dim))))
    c = KVCache.empty(len(lens), cfg.n_kv_heads, capacity, cfg.head_dim, F16)
    c.k[:] = _f16(g.standard_normal(c.k.shape))
    c.v[:] = _f16(g.standard_normal(c.v.shape))
    c.lens[:] = lens
    return wb, c


def test_decoder_layer_is_attention_with_residual_then_mlp():
    acfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    mcfg = MlpConfig(hidden=32, intermediate=48)
    wb, c = _attn(10, acfg, [5, 0], 16)
    aw = LayerWeights.from_bits(wb, F16)
    mw = _mlp_weights(11, 32, 48)
    x = _f16(np.random.default_rng(12).standard_normal((2, 32)))
    c1, c2 = c.copy(), c.copy()
    out = decoder_layer_decode(acfg, aw, mcfg, mw, c1, x)
    # the attention branch alone, plus x, then the MLP on that sum
    a = decode(acfg, aw, c2, x)
    want = mlp(mcfg, mw, a + widen(x, F16))
    assert np.allclose(out, want, rtol=0, atol=1e-12 * np.max(np.abs(want)))
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.lens, c2.lens)
    # zero W_o and zero W_down: the layer is the identity on x
    wb0 = dict(wb, w_o=np.zeros_like(wb["w_o"]))
    mw0 = _mlp_weights(11, 32, 48, zero_down=True)
    assert np.array_equal(decoder_layer_decode(acfg, LayerWeights.from_bits(wb0, F16), mcfg, mw0, c.copy(), x),
                          widen(x, F16))


def test_decoder_layer_verify_rows_equal_sequential_layer_decode():
    acfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    mcfg = MlpConfig(hidden=32, intermediate=48)
    wb, c = _attn(20, acfg, [3, 7], 24)
    aw = LayerWeights.from_bits(wb, F16)
    mw = _mlp_weights(21, 32, 48)
    x = _f16(np.random.default_rng(22).standard_normal((2, 3, 32)))
    c1, c2 = c.copy(), c.copy()
    ov = decoder_layer_verify(acfg, aw, mcfg, mw, c1, x)
    for r in range(3):
        od = decoder_layer_decode(acfg, aw, mcfg, mw, c2, x[:, r, :])
        assert np.max(np.abs(ov[:, r] - od)) < 1e-12 * np.max(np.abs(od))
