"""Pins of the oracle's paged cache (a vLLM-style page table, the engine "Baseten optimizes
Qwen3-ASR 1.7B" names in "Our optimized Qwen3-ASR stack"): the address map against a hand-worked
pool, scatter and gather against a placement built position by position here, the rows a call
appends against where they must land, and a bad page id against its status bit.  A swapped page
index and row, a page-major vs head-major mix-up, an off-by-one at a page boundary or an append
written past its rows fails one of them."""
import numpy as np
import pytest

from oracle import (F16, STATUS_BAD_PAGE, KVCache, LayerWeights, PagedKV, decode, kv_append, mixed, on_pages,
                    verify)

from test_oracle_block import TINY, f16_bits, rand_weights


def test_address_map_hand_worked():
    # P = 2, two pages per slot, four pages; pool value = 10 page + row (one kv head, d = 1)
    pkv = PagedKV.empty(4, 1, 2, 1, [[2, 0], [3, 1]], F16)
    for p in range(4):
        for r in range(2):
            pkv.k[p, 0, r, 0] = 10 * p + r
            pkv.v[p, 0, r, 0] = 100 + 10 * p + r
    c = pkv.gather()
    assert c.k[:, 0, :, 0].tolist() == [[20, 21, 0, 1], [30, 31, 10, 11]]
    assert c.v[:, 0, :, 0].tolist() == [[120, 121, 100, 101], [130, 131, 110, 111]]
    assert pkv.capacity == 4
    assert pkv.locate(1, 3) == (1, 1) and pkv.locate(0, 2) == (0, 0)


def test_head_major_inside_a_page():
    # two kv heads: page p, head g, row r holds 100 p + 10 g + r; slot 0 reads pages 1 then 0
    pkv = PagedKV.empty(2, 2, 3, 1, [[1, 0]], F16)
    for p in range(2):
        for g in range(2):
            for r in range(3):
                pkv.k[p, g, r, 0] = 100 * p + 10 * g + r
    c = pkv.gather()
    assert c.k[0, 0, :, 0].tolist() == [100, 101, 102, 0, 1, 2]
    assert c.k[0, 1, :, 0].tolist() == [110, 111, 112, 10, 11, 12]


def _placed(cont: KVCache, table, P, num_pages):
    """The pool that holds the contiguous cache under `table`, filled position by position."""
    B, nkv, cap, d = cont.k.shape
    k = np.zeros((num_pages, nkv, P, d), np.uint16)
    v = np.zeros_like(k)
    for s in range(B):
        for t in range(cap):
            p = table[s][t // P]
            for g in range(nkv):
                k[p, g, t % P] = cont.k[s, g, t]
                v[p, g, t % P] = cont.v[s, g, t]
    return k, v


def test_scatter_and_gather_invert_each_other():
    g = np.random.default_rng(5)
    B, nkv, P, pps, d = 3, 2, 4, 3, 8
    table = g.permutation(B * pps).reshape(B, pps)
    cont = KVCache.empty(B, nkv, P * pps, d, F16)
    cont.k[:] = g.integers(0, 60000, cont.k.shape)
    cont.v[:] = g.integers(0, 60000, cont.v.shape)
    pkv = PagedKV.empty(B * pps, nkv, P, d, table, F16)
    for s in range(B):
        pkv.scatter_rows(cont, s, 0, P * pps)
    k, v = _placed(cont, table, P, B * pps)
    assert np.array_equal(pkv.k, k) and np.array_equal(pkv.v, v)
    back = pkv.gather()
    assert np.array_equal(back.k, cont.k) and np.array_equal(back.v, cont.v)


def test_append_lands_in_its_pages_and_nowhere_else():
    # P = 2, slot 1 at length 1 appends 3 rows: (page 5, row 1), (page 0, rows 0 and 1)
    pkv = PagedKV.empty(6, 1, 2, 4, [[1, 2, 3], [5, 0, 4]], F16)
    pkv.k[:] = 7
    pkv.v[:] = 9
    pkv.lens[:] = [3, 1]
    kb = np.arange(3 * 4, dtype=np.uint16).reshape(1, 3, 1, 4) + 1000
    vb = kb + 1000
    on_pages(pkv, [1], [3], lambda c: kv_append(c, kb, vb, slots=[1]))
    want_k = np.full((6, 1, 2, 4), 7, np.uint16)
    want_k[5, 0, 1] = kb[0, 0, 0]
    want_k[0, 0, 0] = kb[0, 1, 0]
    want_k[0, 0, 1] = kb[0, 2, 0]
    assert np.array_equal(pkv.k, want_k)
    assert np.array_equal(pkv.v, np.where(want_k == 7, 9, want_k + 1000))
    assert pkv.lens.tolist() == [3, 4] and pkv.status == 0


def test_bad_page_sets_status_and_spares_the_other_sequences():
    pkv = PagedKV.empty(4, 1, 2, 4, [[0, -1], [2, 3]], F16)
    pkv.lens[:] = [1, 1]
    kb = np.full((2, 2, 1, 4), 500, np.uint16)
    on_pages(pkv, [0, 1], [2, 2], lambda c: kv_append(c, kb, kb, slots=[0, 1]))
    assert pkv.status & STATUS_BAD_PAGE
    assert pkv.lens.tolist() == [1, 3]                     # slot 0 needed its page 1 (id -1)
    assert pkv.k[2, 0, 1].tolist() == [500] * 4 and pkv.k[3, 0, 0].tolist() == [500] * 4
    assert not pkv.k[0].any() and not pkv.k[1].any()       # nothing written for slot 0
    ok = PagedKV.empty(4, 1, 2, 4, [[0, -1], [2, 3]], F16)
    ok.lens[:] = [0, 0]
    on_pages(ok, [0], [2], lambda c: kv_append(c, kb[:1], kb[:1], slots=[0]))
    assert ok.status == 0 and ok.lens.tolist() == [2, 0]   # page 1 of slot 0 is never needed


def _paged_fixture(seed, lens, P, pps):
    g = np.random.default_rng(seed)
    B = len(lens)
    num = B * pps + 2
    table = g.permutation(num)[:B * pps].reshape(B, pps)
    cont = KVCache.empty(B, TINY.n_kv_heads, P * pps, TINY.head_dim, F16)
    cont.k[:] = f16_bits(g.standard_normal(cont.k.shape))
    cont.v[:] = f16_bits(g.standard_normal(cont.v.shape))
    cont.lens[:] = lens
    pkv = PagedKV.empty(num, TINY.n_kv_heads, P, TINY.head_dim, table, F16)
    pkv.k[:], pkv.v[:] = _placed(cont, table, P, num)
    pkv.lens[:] = lens
    return g, cont, pkv, table


@pytest.mark.parametrize("lens,P", [([3, 4, 7], 4), ([0, 8, 5], 4), ([2, 9, 1], 3)])
def test_paged_decode_verify_and_mixed_equal_the_contiguous_cache(lens, P):
    """Each call on the pool equals the same call on a contiguous cache holding the same
    positions; the rows it appended sit where the placement puts them (page boundaries crossed
    and started by the appends)."""
    g, cont, pkv, table = _paged_fixture(11 + P, lens, P, 4)
    w = LayerWeights.from_bits(rand_weights(TINY, 12), F16)
    B = len(lens)
    slots = [2, 0, 1]
    x1 = f16_bits(g.standard_normal((B, TINY.hidden)))
    c1, p1 = cont.copy(), pkv.copy()
    want = decode(TINY, w, c1, x1, slots=slots)
    got = on_pages(p1, slots, [1] * B, lambda c: decode(TINY, w, c, x1, slots=slots))
    assert np.array_equal(got, want, equal_nan=True)
    k_pool, v_pool = _placed(c1, table, P, pkv.k.shape[0])
    used = np.unique(table)
    assert np.array_equal(p1.k[used], k_pool[used]) and np.array_equal(p1.v[used], v_pool[used])
    xk = f16_bits(g.standard_normal((B, 3, TINY.hidden)))
    c2, p2 = c1.copy(), p1.copy()
    want = verify(TINY, w, c2, xk, slots=slots)
    got = on_pages(p2, slots, [3] * B, lambda c: verify(TINY, w, c, xk, slots=slots))
    assert np.array_equal(got, want, equal_nan=True)
    sizes = [2, 1, 4]
    xm = f16_bits(g.standard_normal((sum(sizes), TINY.hidden)))
    c3, p3 = c2.copy(), p2.copy()
    want = mixed(TINY, w, c3, xm, sizes, slots=slots)
    got = on_pages(p3, slots, sizes, lambda c: mixed(TINY, w, c, xm, sizes, slots=slots))
    assert np.array_equal(got, want, equal_nan=True)
    k_pool, v_pool = _placed(c3, table, P, pkv.k.shape[0])
    assert np.array_equal(p3.k[used], k_pool[used]) and np.array_equal(p3.v[used], v_pool[used])
    assert p3.lens.tolist() == c3.lens.tolist()


def test_shared_prefix_page_gives_equal_outputs():
    """Two slots whose tables name the same first page and hold equal later rows decode the
    same input to the same output; the shared page is never written (both appends land later)."""
    g = np.random.default_rng(31)
    P = 4
    pkv = PagedKV.empty(5, TINY.n_kv_heads, P, TINY.head_dim, [[0, 1, 2], [0, 3, 4]], F16)
    pkv.k[:] = f16_bits(g.standard_normal(pkv.k.shape))
    pkv.v[:] = f16_bits(g.standard_normal(pkv.v.shape))
    pkv.k[3], pkv.v[3] = pkv.k[1], pkv.v[1]
    pkv.lens[:] = [6, 6]
    shared = pkv.k[0].copy()
    w = LayerWeights.from_bits(rand_weights(TINY, 13), F16)
    x = f16_bits(g.standard_normal((1, TINY.hidden)))
    x2 = np.concatenate([x, x])
    out = on_pages(pkv, [0, 1], [1, 1], lambda c: decode(TINY, w, c, x2, slots=[0, 1]))
    assert np.array_equal(out[0], out[1])
    assert np.array_equal(pkv.k[0], shared)
    assert np.array_equal(pkv.k[1, :, 2], pkv.k[3, :, 2])
