"""Pins of the fp64 oracle against closed forms, invariants and brute force.

Each test is chosen so that a plausible mistake in the oracle fails it: a
dropped or misplaced term of RMSNorm, a wrong rotary pairing, sign or
frequency ladder, a wrong GQA head map, a K/V mix-up or misalignment, a wrong
softmax scale or mask, or an off-by-one in the cache position.
"""
import math

import numpy as np
import pytest

from oracle import (F16, STATUS_CAPACITY, STATUS_CROP_GROW, BlockConfig, KVCache, LayerWeights,
                    decode, kv_append, kv_crop, mixed, rms_norm, rope, verify, widen)

TINY = BlockConfig(hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=8, dtype=F16)


def f16_bits(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def rand_weights(cfg, seed, gain_std=0.02, w_std=0.3):
    g = np.random.default_rng(seed)
    nqkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    bits = dict(
        input_norm_w=f16_bits(1 + gain_std * g.standard_normal(cfg.hidden)),
        w_qkv=f16_bits(w_std * g.standard_normal((nqkv, cfg.hidden))),
        q_norm_w=f16_bits(1 + gain_std * g.standard_normal(cfg.head_dim)),
        k_norm_w=f16_bits(1 + gain_std * g.standard_normal(cfg.head_dim)),
        w_o=f16_bits(w_std * g.standard_normal((cfg.hidden, cfg.n_q_heads * cfg.head_dim))),
    )
    return bits


def rand_cache(cfg, seed, lens, capacity):
    g = np.random.default_rng(seed)
    c = KVCache.empty(len(lens), cfg.n_kv_heads, capacity, cfg.head_dim, cfg.dtype)
    c.k[:] = f16_bits(g.standard_normal(c.k.shape))
    c.v[:] = f16_bits(g.standard_normal(c.v.shape))
    c.lens[:] = lens
    return c


def rel_err(a, b):
    return np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b))


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    g = np.random.default_rng(1).standard_normal(64)
    c = 3.0
    # mean(x^2) of c*1 is c^2
    assert np.allclose(rms_norm(np.full(64, c), g, 1e-6), g * c / math.sqrt(c * c + 1e-6), rtol=1e-15)


def test_rmsnorm_one_hot_divides_by_dimension():
    # x = c e_j: mean(x^2) = c^2 / n, so only entry j survives with gain g_j c / sqrt(c^2/n + eps)
    n, j, c, eps = 128, 37, 0.5, 1e-6
    g = np.random.default_rng(2).standard_normal(n)
    x = np.zeros(n)
    x[j] = c
    h = rms_norm(x, g, eps)
    assert h[j] == pytest.approx(g[j] * c / math.sqrt(c * c / n + eps), rel=1e-15)
    assert np.count_nonzero(h) == 1


def test_rmsnorm_zero_and_eps():
    # all-zero input stays zero; eps alone keeps the denominator finite
    assert np.all(rms_norm(np.zeros(8), np.ones(8), 1e-6) == 0)
    # for a tiny input eps dominates: h ~ x / sqrt(eps)
    x = np.full(8, 1e-9)
    assert rms_norm(x, np.ones(8), 1e-6)[0] == pytest.approx(1e-9 / math.sqrt(1e-18 + 1e-6), rel=1e-12)


# ---------------------------------------------------------------- rotary

def test_rope_position_zero_is_identity():
    u = np.random.default_rng(3).standard_normal((5, 128))
    assert np.array_equal(rope(u, 0, 1e6), u)


def test_rope_preserves_norm_and_composes():
    g = np.random.default_rng(4)
    u = g.standard_normal(128)
    for p1, p2 in [(1, 2), (64, 731), (925, 3000)]:
        r = rope(u, p1 + p2, 1e6)
        assert np.linalg.norm(r) == pytest.approx(np.linalg.norm(u), rel=1e-13)
        assert np.allclose(rope(rope(u, p1, 1e6), p2, 1e6), r, rtol=0, atol=1e-11)


def test_rope_relative_position_identity():
    # <R(m) q, R(n) k> depends only on m - n
    g = np.random.default_rng(5)
    q, k = g.standard_normal(128), g.standard_normal(128)
    for m, n, delta in [(64, 0, 17), (925, 900, 1000), (5, 4000, 3)]:
        s1 = rope(q, m, 1e6) @ rope(k, n, 1e6)
        s2 = rope(q, m + delta, 1e6) @ rope(k, n + delta, 1e6)
        assert s1 == pytest.approx(s2, rel=1e-10, abs=1e-10)


def test_rope_is_complex_rotation_of_half_pairs():
    # (u_t + i u_{t+d/2}) * exp(i angle_t): the rotate-half pairing with a positive sine
    g = np.random.default_rng(6)
    u = g.standard_normal(128)
    r1 = rope(u, 1, 1e6)
    ang = np.angle((r1[:64] + 1j * r1[64:]) / (u[:64] + 1j * u[64:]))      # angle_t at p = 1
    p = 300
    z = (u[:64] + 1j * u[64:]) * np.exp(1j * p * ang)
    assert np.allclose(rope(u, p, 1e6), np.concatenate([z.real, z.imag]), atol=1e-10)


def test_rope_frequency_ladder():
    # angles at p = 1 from unit vectors: omega_0 = 1, a constant ratio between neighbours,
    # and omega_t * omega_{64 - t} = 1 / theta (a geometric ladder from 1 towards 1/theta)
    omega = np.empty(64)
    for t in range(64):
        e = np.zeros(128)
        e[t] = 1.0
        r = rope(e, 1, 1e6)
        omega[t] = math.atan2(r[t + 64], r[t])
    assert omega[0] == pytest.approx(1.0, rel=1e-15)
    ratios = omega[1:] / omega[:-1]
    assert np.allclose(ratios, ratios[0], rtol=1e-12) and ratios[0] < 1
    assert np.allclose(omega[1:64] * omega[63:0:-1], 1e-6, rtol=1e-12)


# ---------------------------------------------------------------- brute force of the whole block

def _brute_decode_row(cfg, wb, kbits, vbits, L, xbits, pos):
    """Scalar loops with math.fsum / math.exp; fp16 only; one row of one sequence."""
    dec = lambda b: float(np.array(b, np.uint16).view(np.float16))
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    x = [dec(b) for b in xbits]
    gin = [dec(b) for b in wb["input_norm_w"]]
    inv = 1.0 / math.sqrt(math.fsum(v * v for v in x) / H + cfg.rms_eps)
    h = [x[j] * gin[j] * inv for j in range(H)]
    W = [[dec(b) for b in row] for row in wb["w_qkv"]]
    qkv = [math.fsum(W[o][j] * h[j] for j in range(H)) for o in range(len(W))]

    def head_norm(vec, gbits):
        gg = [dec(b) for b in gbits]
        iv = 1.0 / math.sqrt(math.fsum(v * v for v in vec) / d + cfg.rms_eps)
        return [vec[j] * gg[j] * iv for j in range(d)]

    def rot(vec):
        out = [0.0] * d
        for t in range(d // 2):
            a = pos * cfg.rope_theta ** (-2.0 * t / d)
            out[t] = vec[t] * math.cos(a) - vec[t + d // 2] * math.sin(a)
            out[t + d // 2] = vec[t + d // 2] * math.cos(a) + vec[t] * math.sin(a)
        return out

    q = [rot(head_norm(qkv[i * d:(i + 1) * d], wb["q_norm_w"])) for i in range(nq)]
    k = [rot(head_norm(qkv[(nq + j) * d:(nq + j + 1) * d], wb["k_norm_w"])) for j in range(nkv)]
    v = [qkv[(nq + nkv + j) * d:(nq + nkv + j + 1) * d] for j in range(nkv)]
    r16 = lambda val: float(np.float16(val))       # numpy's direct nearest-even conversion
    a_all = []
    for i in range(nq):
        g = i * nkv // nq
        keys = [[dec(b) for b in kbits[g][t]] for t in range(L)] + [[r16(val) for val in k[g]]]
        vals = [[dec(b) for b in vbits[g][t]] for t in range(L)] + [[r16(val) for val in v[g]]]
        s = [math.fsum(q[i][c] * keys[t][c] for c in range(d)) / math.sqrt(d) for t in range(L + 1)]
        m = max(s)
        e = [math.exp(st - m) for st in s]
        z = math.fsum(e)
        a_all += [math.fsum(e[t] * vals[t][c] for t in range(L + 1)) / z for c in range(d)]
    Wo = [[dec(b) for b in row] for row in wb["w_o"]]
    return [math.fsum(Wo[o][c] * a_all[c] for c in range(nq * d)) for o in range(H)]


@pytest.mark.parametrize("L,pos", [(0, 0), (1, 1), (3, 3), (6, 6), (5, 40)])
def test_decode_matches_brute_force(L, pos):
    cfg = TINY
    wb = rand_weights(cfg, 10 + L)
    cache = rand_cache(cfg, 20 + L, [L], capacity=8)
    xbits = f16_bits(np.random.default_rng(30 + L).standard_normal((1, cfg.hidden)))
    want = _brute_decode_row(cfg, wb, cache.k[0], cache.v[0], L, xbits[0], pos)
    got = decode(cfg, LayerWeights.from_bits(wb, F16), cache, xbits, positions=[pos])
    assert rel_err(got[0], np.array(want)) < 1e-12
    assert cache.lens[0] == L + 1


def test_empty_cache_output_is_wo_times_repeated_v():
    # with one visible position the softmax weight is 1: a_i = stored v of kv head i // 2,
    # whatever q, k and the position are
    cfg = BlockConfig(hidden=64, n_q_heads=8, n_kv_heads=4, head_dim=16)
    wb = rand_weights(cfg, 40)
    x = f16_bits(np.random.default_rng(41).standard_normal((1, cfg.hidden)))
    outs = []
    for seed, pos in [(0, 0), (1, 77)]:
        w2 = dict(wb)
        g = np.random.default_rng(seed + 100)
        qk_rows = (cfg.n_q_heads + cfg.n_kv_heads) * cfg.head_dim
        w2["w_qkv"] = wb["w_qkv"].copy()
        w2["w_qkv"][:qk_rows] = f16_bits(g.standard_normal((qk_rows, cfg.hidden)))
        c = KVCache.empty(1, cfg.n_kv_heads, 4, cfg.head_dim, F16)
        out = decode(cfg, LayerWeights.from_bits(w2, F16), c, x, positions=[pos])[0]
        v = widen(c.v[0, :, 0, :], F16)                               # [nkv][d] as stored
        rep = np.concatenate([v[i // 2] for i in range(cfg.n_q_heads)])
        assert rel_err(out, widen(wb["w_o"], F16) @ rep) < 1e-13
        outs.append(out)
    assert rel_err(outs[0], outs[1]) < 1e-13


def test_zero_query_gives_mean_of_values():
    cfg = TINY
    wb = rand_weights(cfg, 50)
    wb["w_qkv"][: cfg.n_q_heads * cfg.head_dim] = 0        # q = 0: every score is 0, weights uniform
    L = 5
    cache = rand_cache(cfg, 51, [L], capacity=8)
    x = f16_bits(np.random.default_rng(52).standard_normal((1, cfg.hidden)))
    out = decode(cfg, LayerWeights.from_bits(wb, F16), cache, x)[0]
    V = widen(cache.v[0, :, : L + 1, :], F16)                       # includes the appended row
    a = np.concatenate([V[i // 2].mean(axis=0) for i in range(cfg.n_q_heads)])
    assert rel_err(out, widen(wb["w_o"], F16) @ a) < 1e-13


def test_dominant_key_selects_its_value():
    # every q row of W_q equal to one vector w makes q_raw = c * 1, so after the head norm at
    # position 0 q = sign(c) * g_q (up to eps).  A cached key 20 * sign(c) * g_q then scores
    # about 20 * d / sqrt(d) against O(1) for the others and takes all weight: a_i = V[i // 2][t*].
    cfg = TINY
    d, nq = cfg.head_dim, cfg.n_q_heads
    wb = rand_weights(cfg, 60)
    g = np.random.default_rng(61)
    wrow = f16_bits(g.standard_normal(cfg.hidden))
    wb["w_qkv"][: nq * d] = wrow[None, :]
    L, t_star = 5, 2
    c = rand_cache(cfg, 62, [L], capacity=8)
    x = f16_bits(g.standard_normal((1, cfg.hidden)))
    xs, gin, wv = widen(x[0], F16), widen(wb["input_norm_w"], F16), widen(wrow, F16)
    sign = math.copysign(1.0, math.fsum(wv * gin * xs))
    c.k[0, :, t_star, :] = f16_bits(20.0 * sign * widen(wb["q_norm_w"], F16))[None, :]
    out = decode(cfg, LayerWeights.from_bits(wb, F16), c, x, positions=[0])[0]
    V = widen(c.v[0, :, t_star, :], F16)
    a = np.concatenate([V[i // 2] for i in range(nq)])
    assert rel_err(out, widen(wb["w_o"], F16) @ a) < 1e-12


def test_permuting_cached_positions_keeps_output():
    cfg = TINY
    wb = rand_weights(cfg, 70)
    L = 6
    c1 = rand_cache(cfg, 71, [L], capacity=8)
    c2 = c1.copy()
    perm = np.random.default_rng(72).permutation(L)
    c2.k[0, :, :L] = c1.k[0][:, perm]
    c2.v[0, :, :L] = c1.v[0][:, perm]
    x = f16_bits(np.random.default_rng(73).standard_normal((1, cfg.hidden)))
    w = LayerWeights.from_bits(wb, F16)
    assert rel_err(decode(cfg, w, c2, x)[0], decode(cfg, w, c1, x)[0]) < 1e-13
    # moving only V (not K) changes the output: keys and values are read as pairs
    c3 = c1.copy()
    c3.v[0, :, :L] = c1.v[0][:, perm]
    assert rel_err(decode(cfg, w, c3, x)[0], decode(cfg, w, c1.copy(), x)[0]) > 1e-6


def test_gqa_equals_mha_with_repeated_kv_heads():
    # q head i reads kv head i // (nq / nkv): repeating every kv head twice into an MHA layer
    # (weights and cache) gives the same output
    gqa = TINY
    mha = BlockConfig(hidden=16, n_q_heads=4, n_kv_heads=4, head_dim=8, dtype=F16)
    wb = rand_weights(gqa, 80)
    d, nq = gqa.head_dim, gqa.n_q_heads
    q_rows = wb["w_qkv"][: nq * d]
    k_rows = wb["w_qkv"][nq * d:(nq + 2) * d].reshape(2, d, -1)
    v_rows = wb["w_qkv"][(nq + 2) * d:].reshape(2, d, -1)
    rep = [0, 0, 1, 1]
    wm = dict(wb)
    wm["w_qkv"] = np.concatenate([q_rows, k_rows[rep].reshape(4 * d, -1), v_rows[rep].reshape(4 * d, -1)])
    L = 5
    cg = rand_cache(gqa, 81, [L], capacity=8)
    cm = KVCache.empty(1, 4, 8, d, F16)
    cm.k[0] = cg.k[0][rep]
    cm.v[0] = cg.v[0][rep]
    cm.lens[:] = L
    x = f16_bits(np.random.default_rng(82).standard_normal((1, gqa.hidden)))
    og = decode(gqa, LayerWeights.from_bits(wb, F16), cg, x)[0]
    om = decode(mha, LayerWeights.from_bits(wm, F16), cm, x)[0]
    assert rel_err(og, om) < 1e-13


def test_residual_is_added():
    cfg = TINY
    wb = rand_weights(cfg, 90)
    w = LayerWeights.from_bits(wb, F16)
    c = rand_cache(cfg, 91, [3], capacity=8)
    x = f16_bits(np.random.default_rng(92).standard_normal((1, cfg.hidden)))
    r = f16_bits(np.random.default_rng(93).standard_normal((1, cfg.hidden)))
    o1 = decode(cfg, w, c.copy(), x)
    o2 = decode(cfg, w, c.copy(), x, residual_bits=r)
    assert np.allclose(o2 - o1, widen(r, F16), atol=1e-12)


# ---------------------------------------------------------------- verify, append, crop

@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_verify_block_equals_sequential_decode(k):
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    wb = rand_weights(cfg, 100 + k)
    w = LayerWeights.from_bits(wb, F16)
    lens = [3, 0, 7]
    c1 = rand_cache(cfg, 110 + k, lens, capacity=32)
    c2 = c1.copy()
    x = f16_bits(np.random.default_rng(120 + k).standard_normal((3, k, cfg.hidden)))
    slots = [2, 0, 1]
    ov = verify(cfg, w, c1, x, slots=slots)
    for r in range(k):
        od = decode(cfg, w, c2, x[:, r, :], slots=slots)
        assert rel_err(ov[:, r, :], od) < 1e-12
    assert np.array_equal(c1.lens, c2.lens)
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v)


@pytest.mark.parametrize("a", [0, 1, 3, 4])
def test_crop_after_rejection_equals_never_appended(a):
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    w = LayerWeights.from_bits(rand_weights(cfg, 130), F16)
    L, k = 6, 4
    base = rand_cache(cfg, 131, [L], capacity=16)
    xs = f16_bits(np.random.default_rng(132).standard_normal((1, k, cfg.hidden)))
    xnext = f16_bits(np.random.default_rng(133).standard_normal((1, cfg.hidden)))
    spec = base.copy()
    verify(cfg, w, spec, xs)
    kv_crop([spec], [L + a])
    ref = base.copy()
    if a:
        verify(cfg, w, ref, xs[:, :a, :])
    assert np.array_equal(spec.lens, ref.lens) and spec.status == 0
    assert np.array_equal(spec.k[:, :, : L + a], ref.k[:, :, : L + a])
    o_spec = decode(cfg, w, spec, xnext)
    o_ref = decode(cfg, w, ref, xnext)
    assert np.array_equal(o_spec, o_ref)


def test_append_copies_rows_at_lengths():
    c = KVCache.empty(3, 2, 10, 4, F16)
    c.lens[:] = [1, 5, 0]
    g = np.random.default_rng(140)
    kb = g.integers(0, 2 ** 16, (2, 3, 2, 4)).astype(np.uint16)
    vb = g.integers(0, 2 ** 16, (2, 3, 2, 4)).astype(np.uint16)
    before = c.copy()
    kv_append(c, kb, vb, slots=[2, 0])
    assert c.lens.tolist() == [4, 5, 3]
    assert np.array_equal(c.k[2, :, 0:3], kb[0].transpose(1, 0, 2))
    assert np.array_equal(c.v[0, :, 1:4], vb[1].transpose(1, 0, 2))
    untouched = np.ones(c.k.shape, bool)
    untouched[2, :, 0:3] = False
    untouched[0, :, 1:4] = False
    assert np.array_equal(c.k[untouched], before.k[untouched])


def test_capacity_overflow_and_crop_growth_set_status():
    cfg = TINY
    w = LayerWeights.from_bits(rand_weights(cfg, 150), F16)
    c = rand_cache(cfg, 151, [8, 2], capacity=8)
    x = f16_bits(np.random.default_rng(152).standard_normal((2, cfg.hidden)))
    out = decode(cfg, w, c, x)
    assert np.all(np.isnan(out[0])) and np.all(np.isfinite(out[1]))
    assert c.status == STATUS_CAPACITY and c.lens.tolist() == [8, 3]
    kv_crop([c], [9, 1])
    assert c.lens.tolist() == [8, 1] and c.status == STATUS_CAPACITY | STATUS_CROP_GROW


# ---------------------------------------------------------------- verify's own branches

def _verify_fixture(seed, lens, k, capacity=32):
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    w = LayerWeights.from_bits(rand_weights(cfg, seed), F16)
    c = rand_cache(cfg, seed + 1, lens, capacity=capacity)
    g = np.random.default_rng(seed + 2)
    x = f16_bits(g.standard_normal((len(lens), k, cfg.hidden)))
    r = f16_bits(g.standard_normal((len(lens), k, cfg.hidden)))
    return cfg, w, c, x, r


@pytest.mark.parametrize("k", [1, 3, 5])
def test_verify_explicit_positions_equal_decode_at_p_plus_r(k):
    """Row r of sequence b turns by positions[b] + r: the same rows as k decode steps given the
    positions p_b + r explicitly (decode's explicit positions are pinned by brute force).  The
    positions differ per sequence, so indexing them by slot instead of by sequence fails."""
    lens = [3, 0, 7]
    slots = [2, 0, 1]
    pos = [40, 5, 1000]
    cfg, w, c1, x, _ = _verify_fixture(160 + k, lens, k)
    c2 = c1.copy()
    ov = verify(cfg, w, c1, x, slots=slots, positions=pos)
    for r in range(k):
        od = decode(cfg, w, c2, x[:, r, :], slots=slots, positions=[p + r for p in pos])
        assert rel_err(ov[:, r, :], od) < 1e-12
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v)
    # and the positions matter: the default positions (the lengths) give other rows
    c3 = rand_cache(cfg, 161 + k, lens, capacity=32)
    assert rel_err(verify(cfg, w, c3, x, slots=slots), ov) > 1e-3


@pytest.mark.parametrize("k", [2, 4])
def test_verify_residual_rows_match_decode_with_the_same_residual_rows(k):
    """The residual is [B][k][H]: row r of sequence b gets residual[b][r].  Checked against k
    decode steps each given residual[:, r] (decode's residual is pinned above), and against the
    verify output without residual plus the widened residual."""
    lens = [4, 9]
    cfg, w, c1, x, res = _verify_fixture(170 + k, lens, k)
    c2, c3 = c1.copy(), c1.copy()
    ov = verify(cfg, w, c1, x, residual_bits=res)
    for r in range(k):
        od = decode(cfg, w, c2, x[:, r, :], residual_bits=res[:, r, :])
        assert rel_err(ov[:, r, :], od) < 1e-12
    plain = verify(cfg, w, c3, x)
    assert np.allclose(ov - plain, widen(res, F16), atol=1e-12)


def test_verify_capacity_overflow_skips_that_sequence_only():
    """One sequence whose block would pass the capacity: its k rows are NaN, its length and
    cache rows stay, the capacity bit is set; the other sequences equal a call without it."""
    k, cap = 4, 12
    lens = [5, 9, 8]           # 9 + 4 = 13 > 12 by one row; 8 + 4 = 12 fits exactly
    cfg, w, c, x, _ = _verify_fixture(180, lens, k, capacity=cap)
    before = c.copy()
    out = verify(cfg, w, c, x)
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[[0, 2]]))
    assert c.status == STATUS_CAPACITY
    assert c.lens.tolist() == [9, 9, 12]
    assert np.array_equal(c.k[1], before.k[1]) and np.array_equal(c.v[1], before.v[1])
    keep = [0, 2]
    sub = KVCache(before.k[keep].copy(), before.v[keep].copy(), before.lens[keep].copy(), F16)
    want = verify(cfg, w, sub, x[keep])
    assert np.array_equal(out[keep], want) and sub.status == 0
    assert np.array_equal(c.k[keep], sub.k) and np.array_equal(c.v[keep], sub.v)


# ---------------------------------------------------------------- multi-section rotary

SECTIONS = (16, 24, 24)


def test_mrope_with_equal_components_is_the_one_position_rotary():
    u = np.random.default_rng(300).standard_normal((5, 128))
    for p in (0, 1, 77, 4095):
        assert np.array_equal(rope(u, np.full((5, 3), p), 1e6, SECTIONS), rope(u, np.full(5, p), 1e6))


def test_mrope_pairs_turn_by_their_own_component():
    """Scalar loop over the pairs: pair t turns by p[c(t)] * theta^(-2t/d)."""
    g = np.random.default_rng(301)
    u = g.standard_normal(128)
    p3 = np.array([5, 900, 33])
    out = rope(u[None], p3[None], 1e6, SECTIONS)[0]
    for t in range(64):
        c = 0 if t < 16 else (1 if t < 40 else 2)
        ang = p3[c] * 1e6 ** (-2.0 * t / 128)
        assert out[t] == pytest.approx(u[t] * math.cos(ang) - u[t + 64] * math.sin(ang), abs=1e-12)
        assert out[t + 64] == pytest.approx(u[t + 64] * math.cos(ang) + u[t] * math.sin(ang), abs=1e-12)
    # a section of all 64 pairs is the one-position rotary of that component
    assert np.allclose(rope(u[None], p3[None], 1e6, (64, 0, 0))[0], rope(u, 5, 1e6), atol=1e-15)


def test_mrope_scores_depend_on_each_component_difference_only():
    """Shifting all three components of query and key by the same per-component offsets keeps
    q . k (each section is a rotation by the difference of its own components)."""
    g = np.random.default_rng(302)
    q, k = g.standard_normal(128), g.standard_normal(128)
    m, n, delta = np.array([10, 20, 30]), np.array([3, 7, 100]), np.array([5, -9, 1000])
    s1 = rope(q[None], m[None], 1e6, SECTIONS)[0] @ rope(k[None], n[None], 1e6, SECTIONS)[0]
    s2 = rope(q[None], (m + delta)[None], 1e6, SECTIONS)[0] @ rope(k[None], (n + delta)[None], 1e6, SECTIONS)[0]
    assert abs(s1 - s2) < 1e-10


def test_mrope_verify_equals_sequential_decode():
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16, mrope_sections=(2, 3, 3))
    wb = rand_weights(cfg, 310)
    w = LayerWeights.from_bits(wb, F16)
    c1 = rand_cache(cfg, 311, [3, 6], capacity=16)
    c2 = c1.copy()
    x = f16_bits(np.random.default_rng(312).standard_normal((2, 3, cfg.hidden)))
    pos3 = np.array([[10, 4], [200, 7], [31, 9]])
    ov = verify(cfg, w, c1, x, positions=pos3)
    for r in range(3):
        od = decode(cfg, w, c2, x[:, r, :], positions=pos3 + r)
        assert rel_err(ov[:, r], od) < 1e-12
    # and it differs from the one-position rotary at component 0
    c3 = rand_cache(cfg, 311, [3, 6], capacity=16)
    one = verify(BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16), w, c3, x, positions=pos3[0])
    assert rel_err(one, ov) > 1e-3


# ---------------------------------------------------------------- mixed decode rows and verify blocks

def _sequential_decode(cfg, w, cache, x, sizes, slots, positions, residual):
    """Each sequence's block as single-token decode steps of that sequence alone."""
    out = np.empty((sum(sizes), cfg.hidden))
    row = 0
    for b, n in enumerate(sizes):
        for r in range(n):
            if positions is None:
                pos = None
            elif cfg.mrope_sections:
                pos = np.asarray(positions)[:, b:b + 1] + r
            else:
                pos = [positions[b] + r]
            res = residual[row + r:row + r + 1] if residual is not None else None
            out[row + r] = decode(cfg, w, cache, x[row + r:row + r + 1], slots=[slots[b]], positions=pos,
                                  residual_bits=res)[0]
        row += n
    return out


@pytest.mark.parametrize("sections", [(), (2, 3, 3)])
def test_mixed_blocks_equal_sequential_decode_per_sequence(sections):
    """Rows of every sequence in a mixed call (block sizes 1, 4, 2, 1, 3; permuted slots, explicit
    positions and a residual) equal that sequence's tokens decoded one by one; the cache rows and
    lengths agree too.  A wrong row offset, slot or position lookup fails it."""
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16, mrope_sections=sections)
    w = LayerWeights.from_bits(rand_weights(cfg, 400), F16)
    sizes = [1, 4, 2, 1, 3]
    slots = [3, 0, 4, 1, 2]
    c1 = rand_cache(cfg, 401, [5, 0, 9, 2, 11], capacity=24)
    c2 = c1.copy()
    rows = sum(sizes)
    x = f16_bits(np.random.default_rng(402).standard_normal((rows, cfg.hidden)))
    res = f16_bits(np.random.default_rng(403).standard_normal((rows, cfg.hidden)))
    pos = np.array([[40, 7, 300, 2, 19], [8, 50, 1, 90, 3], [61, 0, 17, 4, 200]]) if sections else [40, 7, 300, 2, 19]
    got = mixed(cfg, w, c1, x, sizes, slots=slots, positions=pos, residual_bits=res)
    want = _sequential_decode(cfg, w, c2, x, sizes, slots, pos, res)
    assert rel_err(got, want) < 1e-12
    assert np.array_equal(c1.lens, c2.lens) and np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v)
    assert [int(c1.lens[slots[b]]) for b in range(5)] == [l + n for l, n in zip([2, 5, 11, 0, 9], sizes)]


def test_mixed_blocks_of_one_row_are_a_decode_step():
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    w = LayerWeights.from_bits(rand_weights(cfg, 410), F16)
    c1 = rand_cache(cfg, 411, [4, 0, 6], capacity=16)
    c2 = c1.copy()
    x = f16_bits(np.random.default_rng(412).standard_normal((3, cfg.hidden)))
    got = mixed(cfg, w, c1, x, [1, 1, 1], slots=[1, 2, 0])
    want = decode(cfg, w, c2, x, slots=[1, 2, 0])
    assert np.array_equal(got, want)
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.lens, c2.lens)


def test_mixed_capacity_overflow_skips_that_sequence_only():
    cfg = BlockConfig(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=16)
    w = LayerWeights.from_bits(rand_weights(cfg, 420), F16)
    c1 = rand_cache(cfg, 421, [3, 14, 5], capacity=16)
    c2 = c1.copy()
    x = f16_bits(np.random.default_rng(422).standard_normal((2 + 3 + 4, cfg.hidden)))
    got = mixed(cfg, w, c1, x, [2, 3, 4])          # sequence 1: 14 + 3 > 16
    assert np.all(np.isnan(got[2:5])) and np.all(np.isfinite(got[:2])) and np.all(np.isfinite(got[5:]))
    assert c1.status == STATUS_CAPACITY and c1.lens.tolist() == [5, 14, 9]
    assert np.array_equal(c1.k[1], c2.k[1])
    want0 = verify(cfg, w, c2, x[None, :2], slots=[0])[0]
    assert rel_err(got[:2], want0) < 1e-12
