"""Pins of the oracle's FP8 (E4M3) cache: the code table, the saturating
round-to-nearest-even conversion, an independent encoder, and attention over an
FP8 cache against brute force and the verify / crop invariants.

E4M3 here is the 8-bit float with 1 sign bit, 4 exponent bits (bias 7) and 3
mantissa bits, no infinities and one NaN pattern per sign (the FP8 KV-cache
format of "Baseten optimizes Qwen3-ASR 1.7B", section "KV cache quantization";
the layout is a reading, that page names only FP8)."""
import math

import numpy as np
import pytest

from oracle import (E4M3, F16, BlockConfig, KVCache, LayerWeights, decode, e4m3_value, kv_crop, rne_e4m3, verify,
                    widen)
from synth import inputs as si


def test_code_table_landmarks():
    v = e4m3_value(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9          # subnormals m * 2^-9
    assert v[0x08] == 2.0 ** -6                                        # smallest normal
    assert v[0x38] == 1.0 and v[0x3F] == 1.875 and v[0x40] == 2.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0                      # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])                     # the only NaNs
    assert np.isnan(v).sum() == 2
    assert np.all(np.diff(v[:0x7F]) > 0)                               # 0x00 .. 0x7E ascending
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(rne_e4m3(e4m3_value(codes)), codes)


def test_midpoints_tie_to_even_and_quarter_points_go_to_nearest():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo, hi = e4m3_value(codes), e4m3_value(codes + 1)
    mid = (lo + hi) / 2
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(rne_e4m3(mid), even)
    assert np.array_equal(rne_e4m3(lo + (hi - lo) / 4), codes)
    assert np.array_equal(rne_e4m3(lo + 3 * (hi - lo) / 4), codes + 1)
    assert np.array_equal(rne_e4m3(-mid), even | 0x80)
    assert rne_e4m3(np.array([2.0 ** -10]))[0] == 0x00                  # tie between 0 and 2^-9
    assert rne_e4m3(np.array([3 * 2.0 ** -10]))[0] == 0x02              # tie between 1 and 2 (x 2^-9)


def test_saturation_nan_and_signed_zero():
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, math.inf])
    assert np.all(rne_e4m3(big) == 0x7E) and np.all(rne_e4m3(-big) == 0xFE)
    assert rne_e4m3(np.array([math.nan]))[0] == 0x7F
    assert rne_e4m3(np.array([-0.0]))[0] == 0x80 and rne_e4m3(np.array([0.0]))[0] == 0x00


def test_independent_encoder_agrees():
    g = np.random.default_rng(7)
    for scale in (2.0 ** -12, 2.0 ** -8, 1.0, 16.0, 200.0):
        a = g.standard_normal(200_000) * scale
        assert np.array_equal(si.to_e4m3_codes(a), rne_e4m3(a))


TINY = BlockConfig(hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=8, dtype=F16)


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def _fixture(seed, lens, capacity, cfg=TINY):
    g = np.random.default_rng(seed)
    nqkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    wb = dict(input_norm_w=_f16(1 + 0.02 * g.standard_normal(cfg.hidden)),
              w_qkv=_f16(0.3 * g.standard_normal((nqkv, cfg.hidden))),
              q_norm_w=_f16(1 + 0.02 * g.standard_normal(cfg.head_dim)),
              k_norm_w=_f16(1 + 0.02 * g.standard_normal(cfg.head_dim)),
              w_o=_f16(0.3 * g.standard_normal((cfg.hidden, cfg.n_q_heads * cfg.head_dim))))
    ks = np.array([0.05, 0.08][:cfg.n_kv_heads], np.float32)
    vs = np.array([0.07, 0.03][:cfg.n_kv_heads], np.float32)
    c = KVCache.empty(len(lens), cfg.n_kv_heads, capacity, cfg.head_dim, E4M3, ks, vs)
    c.k[:] = rne_e4m3(g.standard_normal(c.k.shape) / 0.06)
    c.v[:] = rne_e4m3(g.standard_normal(c.v.shape) / 0.06)
    c.lens[:] = lens
    return LayerWeights.from_bits(wb, F16), c, g


@pytest.mark.parametrize("L", [0, 1, 5])
def test_fp8_cache_decode_matches_brute_force(L):
    """Scalar loops over the definition, with the cache read as scale * code value and the new
    row stored as the code nearest to value / scale."""
    cfg = TINY
    w, c, g = _fixture(200 + L, [L], 8)
    x = _f16(g.standard_normal((1, cfg.hidden)))
    ref = c.copy()
    out = decode(cfg, w, c, x)[0]
    xv = widen(x, F16)[0]
    ms = math.fsum(v * v for v in xv) / cfg.hidden
    h = [xv[i] * w.input_norm_w[i] / math.sqrt(ms + cfg.rms_eps) for i in range(cfg.hidden)]
    qkv = [math.fsum(w.w_qkv[o, i] * h[i] for i in range(cfg.hidden)) for o in range(w.w_qkv.shape[0])]
    d, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads

    def norm_rope(u, gain):
        ms = math.fsum(a * a for a in u) / d
        u = [u[t] * gain[t] / math.sqrt(ms + cfg.rms_eps) for t in range(d)]
        r = list(u)
        for t in range(d // 2):
            ang = L * cfg.rope_theta ** (-2.0 * t / d)
            r[t] = u[t] * math.cos(ang) - u[t + d // 2] * math.sin(ang)
            r[t + d // 2] = u[t + d // 2] * math.cos(ang) + u[t] * math.sin(ang)
        return r
    qs = [norm_rope(qkv[i * d:(i + 1) * d], w.q_norm_w) for i in range(nq)]
    ks = [norm_rope(qkv[(nq + j) * d:(nq + j + 1) * d], w.k_norm_w) for j in range(nkv)]
    vs = [qkv[(nq + nkv + j) * d:(nq + nkv + j + 1) * d] for j in range(nkv)]
    att = []
    for i in range(nq):
        j = i // (nq // nkv)
        keys = [[ref.k_scale[j] * float(e4m3_value(np.uint8(ref.k[0, j, t, e]))) for e in range(d)] for t in range(L)]
        vals = [[ref.v_scale[j] * float(e4m3_value(np.uint8(ref.v[0, j, t, e]))) for e in range(d)] for t in range(L)]
        kq = [float(e4m3_value(rne_e4m3(np.array([ks[j][e] / float(ref.k_scale[j])]))[0])) * ref.k_scale[j] for e in range(d)]
        vq = [float(e4m3_value(rne_e4m3(np.array([vs[j][e] / float(ref.v_scale[j])]))[0])) * ref.v_scale[j] for e in range(d)]
        keys.append(kq)
        vals.append(vq)
        sc = [math.fsum(qs[i][e] * kk[e] for e in range(d)) / math.sqrt(d) for kk in keys]
        m = max(sc)
        ex = [math.exp(s_ - m) for s_ in sc]
        z = math.fsum(ex)
        att.extend(math.fsum(ex[t] / z * vals[t][e] for t in range(len(keys))) for e in range(d))
    want = [math.fsum(w.w_o[o, a] * att[a] for a in range(len(att))) for o in range(cfg.hidden)]
    assert np.max(np.abs(out - want)) / np.sqrt(np.mean(np.square(want))) < 1e-12
    assert c.k.dtype == np.uint8 and c.lens[0] == L + 1


@pytest.mark.parametrize("k", [1, 3, 4])
def test_fp8_verify_equals_sequential_decode(k):
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    w, c1, g = _fixture(210 + k, [3, 0, 9], 24, cfg)
    c2 = c1.copy()
    x = _f16(g.standard_normal((3, k, cfg.hidden)))
    ov = verify(cfg, w, c1, x, slots=[1, 2, 0])
    for r in range(k):
        od = decode(cfg, w, c2, x[:, r, :], slots=[1, 2, 0])
        assert np.max(np.abs(ov[:, r] - od)) / np.sqrt(np.mean(od ** 2)) < 1e-12
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v) and np.array_equal(c1.lens, c2.lens)


def test_fp8_crop_after_rejection_equals_never_appended():
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    w, base, g = _fixture(220, [6], 16, cfg)
    xs = _f16(g.standard_normal((1, 4, cfg.hidden)))
    xn = _f16(g.standard_normal((1, cfg.hidden)))
    spec = base.copy()
    verify(cfg, w, spec, xs)
    kv_crop([spec], [8])
    ref = base.copy()
    verify(cfg, w, ref, xs[:, :2, :])
    assert np.array_equal(decode(cfg, w, spec, xn), decode(cfg, w, ref, xn))


def test_synthetic_fp8_rows_are_the_16bit_draws_divided_by_the_scales():
    ks, vs = si.kv_scales(4, 0)
    kc, vc = si.kv_rows_e4m3(4, 0, 3, 10, ks, vs)
    k16, _ = si.kv_rows(4, 0, 3, 10, si.BF16)
    assert kc.dtype == np.uint8 and kc.shape == (8, 10, 128)
    # the same draws: the decoded fp8 rows are within half an E4M3 step of the bf16 rows
    kv = e4m3_value(kc) * ks.astype(np.float64)[:, None, None]
    kb = widen(k16, si.BF16)
    assert np.max(np.abs(kv - kb) / np.maximum(np.abs(kb), 2.0 ** -6 * ks.max())) < 2.0 ** -3
