"""GPU parity of layer calls on a paged KV cache (a pool of fixed-size pages addressed through a
per-sequence page table, the cache of the vLLM engine "Baseten optimizes Qwen3-ASR 1.7B" starts
its stack from, section "Our optimized Qwen3-ASR stack") against the oracle's paged view, through
the C ABI: decode, verify and mixed calls of every GQA group, page sizes 16 .. 256 with appends
that start and cross pages, shuffled page tables, a shared prefix page, the prefill copy, the
whole decoder layer, bit-identity with the contiguous cache on the same kernel, and a table entry
outside the pool."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import (TOL, SeededLayer, check_rounded_rows, device_cache, fill_cache, oracle_cache, rel_err, tdt,
                        to_bits, to_dev)
from test_gpu_mlp import SeededMlp

pytestmark = pytest.mark.gpu


def _i32(v):
    return None if v is None else torch.tensor(np.asarray(v, np.int32).ravel(), dtype=torch.int32, device="cuda")


def paged_pair(stream, lens, P, pps, dtype, nkv=8, spare=3):
    """An oracle paged cache holding seeded rows below each length, in the pages of a shuffled
    table (spare pages outside every table hold seeded noise), and the same pool on the device."""
    B = len(lens)
    num = B * pps + spare
    table = si.page_table(stream, B, pps, num)
    kb, vb = fill_cache(stream, 0, lens, P * pps, dtype, nkv=nkv)
    cont = oracle_cache(kb, vb, lens, dtype)
    ref = oracle.PagedKV.empty(num, nkv, P, 128, table, dtype)
    free = sorted(set(range(num)) - set(table.ravel().tolist()))
    ref.k[free] = si.normal_bits(stream, 1, si.T_KCACHE, 0, (len(free), nkv, P, 128), 1.0, 0.0, dtype)
    ref.v[free] = si.normal_bits(stream, 1, si.T_VCACHE, 0, (len(free), nkv, P, 128), 1.0, 0.0, dtype)
    for s in range(B):
        ref.scatter_rows(cont, s, 0, P * pps)
    ref.lens[:] = lens
    kv = ga.KVLayer(to_dev(ref.k, dtype), to_dev(ref.v, dtype), _i32(lens),
                    torch.zeros(1, dtype=torch.int32, device="cuda"), block_table=_i32(table).view(B, pps))
    return kv, ref


def run_call(L, cfg, kv, xb, sizes, dtype, slots=None, positions=None, residual=None):
    """decode (all sizes 1), verify (all equal) or mixed, fp32 out [rows][H]."""
    rows, H = xb.shape
    B = len(sizes)
    out = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    ws = ga.alloc_workspace(cfg, rows, kv.capacity)
    x = to_dev(xb, dtype)
    res = None if residual is None else to_dev(residual, dtype)
    if all(n == 1 for n in sizes):
        ga.layer_decode(cfg, L.dev, kv, x, out, ws, slots=_i32(slots), positions=_i32(positions), residual=res)
    elif len(set(sizes)) == 1:
        k = sizes[0]
        ga.layer_verify(cfg, L.dev, kv, x.view(B, k, H), out.view(B, k, H), ws, slots=_i32(slots),
                        positions=_i32(positions), residual=None if res is None else res.view(B, k, H))
    else:
        ga.layer_mixed(cfg, L.dev, kv, x, sizes, out, ws, slots=_i32(slots), positions=_i32(positions), residual=res)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_call(L, ocfg, ref, xb, sizes, slots=None, positions=None, residual=None):
    B = len(sizes)
    slots_l = list(range(B)) if slots is None else list(slots)

    def op(c):
        if all(n == 1 for n in sizes):
            return oracle.decode(ocfg, L.ref, c, xb, slots=slots_l, positions=positions, residual_bits=residual)
        if len(set(sizes)) == 1:
            k = sizes[0]
            return oracle.verify(ocfg, L.ref, c, xb.reshape(B, k, -1), slots=slots_l, positions=positions,
                                 residual_bits=None if residual is None else residual.reshape(B, k, -1)
                                 ).reshape(B * k, -1)
        return oracle.mixed(ocfg, L.ref, c, xb, sizes, slots=slots_l, positions=positions, residual_bits=residual)

    return oracle.on_pages(ref, slots_l, sizes, op)


def check_pool(kv, ref, before_k, before_v, dtype):
    """Appended rows within one unit of the oracle's rounding; every other pool row unchanged."""
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    changed = (ref.k != before_k).any(axis=-1) | (ref.v != before_v).any(axis=-1)
    # rows the oracle wrote (a row may be rewritten with its own bits: compare the rest exactly)
    mask = np.zeros(changed.shape, bool)
    for s in range(ref.table.shape[0]):
        for t in range(int(ref.lens[s])):
            p, r = ref.locate(s, t)
            if p is not None:
                mask[p, :, r] |= changed[p, :, r]
    for p, g, r in zip(*np.nonzero(mask)):
        check_rounded_rows(kg[p, g, r], ref.k[p, g, r], dtype)
        check_rounded_rows(vg[p, g, r], ref.v[p, g, r], dtype)
    keep = ~mask
    assert np.array_equal(kg[keep], ref.k[keep]) and np.array_equal(vg[keep], ref.v[keep])


CASES = {
    # name: (n_q_heads, n_kv_heads, block sizes, committed lengths, page size)
    "decode_bs1_p16": (16, 8, [1], [925], 16),
    "decode_b8_p64": (16, 8, [1] * 8, [64, 0, 925, 127, 1, 300, 63, 500], 64),
    "verify_k4_p32": (16, 8, [4] * 4, [30, 95, 0, 300], 32),
    "verify_k16_p16": (16, 8, [16] * 3, [16, 250, 7], 16),
    "mixed_g2_p64": (16, 8, [1, 4, 8, 1, 16, 2, 1], [30, 0, 250, 129, 7, 64, 283], 64),
    "mixed_g4_p128": (16, 4, [3, 1, 1, 7, 2], [100, 5, 260, 33, 127], 128),
    "mixed_g8_p256": (16, 2, [5, 1, 2, 9], [12, 290, 0, 251], 256),
    "mixed_g1_p16": (8, 8, [1, 2, 6, 1, 1], [61, 3, 199, 0, 240], 16),
    "rows140_p32": (16, 8, [9, 1, 16, 4, 12, 7, 1, 16, 3, 10, 14, 2, 8, 16, 5, 16],
                    [150, 193, 236, 279, 0, 280, 231, 120, 100, 50, 283, 270, 17, 1, 90, 200], 32),
}


@pytest.mark.parametrize("dtype", [si.BF16, si.F16])
@pytest.mark.parametrize("case", sorted(CASES))
def test_paged_vs_oracle(case, dtype):
    """Reversed slots, explicit positions and a residual: outputs, the appended rows in their
    pages, every other pool row (spare pages included) untouched, the lengths."""
    nq, nkv, sizes, lens, P = CASES[case]
    B, rows = len(sizes), sum(sizes)
    pps = (max(l + n for l, n in zip(lens, sizes)) + P - 1) // P + 1
    seed = 80 + sorted(CASES).index(case)
    slots = list(range(B))[::-1]
    L = SeededLayer(seed, 0, 1024, dtype, nq=nq, nkv=nkv)
    kv, ref = paged_pair(seed, [lens[slots.index(s)] for s in range(B)], P, pps, dtype, nkv=nkv)
    before_k, before_v = ref.k.copy(), ref.v.copy()
    xb = si.activations(seed, 0, 0, rows, 1024, dtype)
    res = si.residual(seed, 0, 0, rows, 1024, dtype)
    pos = [7 * b + 1000 * (b % 2) for b in range(B)]
    ocfg = oracle.BlockConfig(hidden=1024, n_q_heads=nq, n_kv_heads=nkv, dtype=dtype)
    print(f"paged {case} {dtype} P={P} pps={pps}", flush=True)
    got = run_call(L, ga.config(dtype=dtype, n_q_heads=nq, n_kv_heads=nkv), kv, xb, sizes, dtype, slots=slots,
                   positions=pos, residual=res)
    want = oracle_call(L, ocfg, ref, xb, sizes, slots=slots, positions=pos, residual=res)
    err = rel_err(got, want)
    print(f"  err {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == ref.lens.tolist()
    assert kv.status.item() == 0 and ref.status == 0
    check_pool(kv, ref, before_k, before_v, dtype)


@pytest.mark.parametrize("nq,nkv,sizes,P", [(16, 2, [3, 5, 1, 7], 16), (8, 8, [1] * 6, 64), (8, 8, [4] * 3, 32),
                                            (16, 8, [1] * 6, 16), (16, 4, [2, 5, 1, 3], 64), (16, 8, [1, 1, 8], 32),
                                            (16, 8, [1], 64), (16, 8, [1, 1, 1], 16), (16, 2, [4], 32),
                                            (8, 8, [2, 2], 16)])
def test_paged_equals_the_contiguous_cache_on_the_same_kernel(nq, nkv, sizes, P):
    """The paged call runs the contiguous call's kernel with another address map (the chunked
    kernel for GQA groups 1 and 8, the equal-share kernel for groups 2 and 4, the few-row kernel
    for up to 4 rows; decode, verify and mixed rows), so it gives the same bits: output and
    appended rows alike."""
    dtype = si.BF16
    B, rows = len(sizes), sum(sizes)
    lens = [300, 17, 0, 128, 64, 255][:B]
    pps = 320 // P
    L = SeededLayer(95, 0, 1024, dtype, nq=nq, nkv=nkv)
    kv, ref = paged_pair(95, lens, P, pps, dtype, nkv=nkv)
    kb, vb = fill_cache(95, 0, lens, P * pps, dtype, nkv=nkv)
    kvc = device_cache(kb, vb, lens, dtype)
    xb = si.activations(95, 0, 0, rows, 1024, dtype)
    cfg = ga.config(dtype=dtype, n_q_heads=nq, n_kv_heads=nkv, kv_split=P)
    a = run_call(L, cfg, kv, xb, sizes, dtype)
    c = run_call(L, cfg, kvc, xb, sizes, dtype)
    assert np.array_equal(a, c)
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    kc, vc = to_bits(kvc.k), to_bits(kvc.v)
    for s, n in enumerate(sizes):
        for t in range(lens[s], lens[s] + n):
            p, r = ref.locate(s, t)
            assert np.array_equal(kg[p, :, r], kc[s, :, t]) and np.array_equal(vg[p, :, r], vc[s, :, t])


def test_paged_shared_prefix_pages():
    """Four sequences whose tables name the same two prompt pages, each with its own later
    pages: outputs against the oracle, and the shared pages never written."""
    dtype, P = si.F16, 64
    L = SeededLayer(96, 0, 1024, dtype)
    B, pps = 4, 6
    prompt = 128                                          # two full shared pages
    lens = [prompt + d for d in (5, 40, 0, 63)]
    table = si.page_table(96, B, pps, B * pps)
    table[:, :2] = table[0, :2]                           # every sequence reads sequence 0's prompt pages
    num = B * pps
    ref = oracle.PagedKV.empty(num, 8, P, 128, table, dtype)
    ref.k[:] = si.normal_bits(96, 2, si.T_KCACHE, 0, ref.k.shape, 1.0, 0.0, dtype)
    ref.v[:] = si.normal_bits(96, 2, si.T_VCACHE, 0, ref.v.shape, 1.0, 0.0, dtype)
    ref.lens[:] = lens
    shared = [int(p) for p in table[0, :2]]
    keep_k, keep_v = ref.k[shared].copy(), ref.v[shared].copy()
    kv = ga.KVLayer(to_dev(ref.k, dtype), to_dev(ref.v, dtype), _i32(lens),
                    torch.zeros(1, dtype=torch.int32, device="cuda"), block_table=_i32(table).view(B, pps))
    xb = si.activations(96, 0, 0, B, 1024, dtype)
    got = run_call(L, ga.config(dtype=dtype), kv, xb, [1] * B, dtype)
    want = oracle_call(L, L.ocfg, ref, xb, [1] * B)
    err = rel_err(got, want)
    print(f"shared prefix: {err:.3e}")
    assert err < TOL[dtype]
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    assert np.array_equal(kg[shared], keep_k) and np.array_equal(vg[shared], keep_v)
    assert kv.lens.cpu().tolist() == [l + 1 for l in lens]


@pytest.mark.parametrize("n,P", [(1, 16), (5, 16), (40, 32)])
def test_paged_append_is_bit_exact(n, P):
    """The prefill copy into pages: bit for bit the oracle's placement, nothing else touched."""
    dtype = si.BF16
    lens = [15, 0, 33, 100]
    B = len(lens)
    pps = (max(lens) + n + P - 1) // P
    kv, ref = paged_pair(97, lens, P, pps, dtype)
    g = np.random.default_rng(97)
    kn = si.to_bits(g.standard_normal((B, n, 8, 128)), dtype)
    vn = si.to_bits(g.standard_normal((B, n, 8, 128)), dtype)
    slots = [2, 0, 3, 1]
    ga.kv_append(kv, to_dev(kn, dtype), to_dev(vn, dtype), slots=_i32(slots))
    torch.cuda.synchronize()
    oracle.on_pages(ref, slots, [n] * B, lambda c: oracle.kv_append(c, kn, vn, slots=slots))
    assert np.array_equal(to_bits(kv.k), ref.k) and np.array_equal(to_bits(kv.v), ref.v)
    assert kv.lens.cpu().tolist() == ref.lens.tolist() and kv.status.item() == 0


def test_paged_decoder_layer_vs_oracle():
    dtype, P = si.BF16, 32
    sizes = [1, 3, 1, 8]
    lens = [200, 31, 0, 96]
    B, rows = len(sizes), sum(sizes)
    pps = 8
    L = SeededLayer(98, 0, 1024, dtype)
    M = SeededMlp(98, 0, 1024, 3072, dtype)
    kv, ref = paged_pair(98, lens, P, pps, dtype)
    xb = si.activations(98, 0, 0, rows, 1024, dtype)
    acfg, mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype)
    out = torch.empty((rows, 1024), dtype=torch.float32, device="cuda")
    ws = ga.decoder_layer_workspace(acfg, mcfg, rows, kv.capacity)
    ga.decoder_layer_mixed(acfg, L.dev, mcfg, M.dev, kv, to_dev(xb, dtype), sizes, out, ws)
    torch.cuda.synchronize()
    want = oracle.on_pages(ref, range(B), sizes, lambda c: oracle.decoder_layer_mixed(L.ocfg, L.ref, M.ocfg, M.ref, c,
                                                                                      xb, sizes))
    err = rel_err(out.cpu().numpy(), want)
    print(f"paged decoder layer: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + n for l, n in zip(lens, sizes)]


@pytest.mark.parametrize("bad", [-3, 1 << 20])
def test_paged_bad_page_id_sets_status_and_spares_the_others(bad):
    """A table entry outside the pool for a page sequence 1 needs: the status bit, no access
    outside the pool (the kernels replace the id), the other sequences' outputs, appended rows
    and every page they do not own untouched."""
    dtype, P = si.F16, 16
    sizes, lens = [1, 4, 2], [40, 30, 70]
    B, rows = len(sizes), sum(sizes)
    pps = 6
    L = SeededLayer(99, 0, 1024, dtype)
    kv, ref = paged_pair(99, lens, P, pps, dtype)
    table = ref.table.copy()
    table[1, 1] = bad                                     # positions 16 .. 31 of sequence 1
    ref.table = table
    kv.block_table.copy_(_i32(table).view(B, pps))
    before_k, before_v = ref.k.copy(), ref.v.copy()
    xb = si.activations(99, 0, 0, rows, 1024, dtype)
    got = run_call(L, ga.config(dtype=dtype), kv, xb, sizes, dtype)
    want = oracle_call(L, L.ocfg, ref, xb, sizes)
    assert kv.status.item() & ga.STATUS_BAD_PAGE and ref.status & oracle.STATUS_BAD_PAGE
    ok = np.r_[0:1, 5:7]                                  # rows of sequences 0 and 2
    assert rel_err(got[ok], want[ok]) < TOL[dtype]
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    own1 = [int(p) for p in table[1] if 0 <= p < ref.k.shape[0]]
    others = [p for p in range(ref.k.shape[0]) if p not in own1]
    for s in (0, 2):
        for t in range(lens[s], lens[s] + sizes[s]):
            p, r = ref.locate(s, t)
            check_rounded_rows(kg[p, :, r], ref.k[p, :, r], dtype)
    written = {ref.locate(s, t)[0] for s in (0, 2) for t in range(lens[s], lens[s] + sizes[s])}
    for p in others:
        if p not in written:
            assert np.array_equal(kg[p], before_k[p]) and np.array_equal(vg[p], before_v[p])
    # the prefill copy on the same table: the status bit, and no row written for the bad page
    kv.status.zero_()
    kn = si.to_bits(np.random.default_rng(99).standard_normal((1, 20, 8, 128)), dtype)
    pool_k = to_bits(kv.k)
    kv.lens.copy_(_i32([0, 0, 0]))
    ga.kv_append(kv, to_dev(kn, dtype), to_dev(kn, dtype), slots=_i32([1]))
    torch.cuda.synchronize()
    assert kv.status.item() & ga.STATUS_BAD_PAGE
    kg2 = to_bits(kv.k)
    p0 = int(table[1, 0])
    assert np.array_equal(kg2[p0, :, :16], kn[0, :16].transpose(1, 0, 2))
    rest = [p for p in range(ref.k.shape[0]) if p != p0]
    assert np.array_equal(kg2[rest], pool_k[rest])


def test_paged_graph_replays_and_workspace_free_decode():
    """Paged decode steps captured in a HIP graph and replayed (a crop back to the start and new
    inputs between replays) leave the eager calls' outputs, pool bits and lengths; the
    workspace-free decode entry gives the decode entry's bits on a paged cache (5 rows on the
    many-row kernels, then 2 rows on the few-row ones)."""
    dtype, P = si.BF16, 16
    lens = [40, 300, 7, 129, 64]
    B, pps = len(lens), 320 // 16
    L = SeededLayer(101, 0, 1024, dtype)
    cfg = ga.config(dtype=dtype)
    ws = ga.alloc_workspace(cfg, B, pps * P)
    xs = [to_dev(si.activations(101, 0, r, B, 1024, dtype), dtype) for r in range(3)]
    x = torch.empty((B, 1024), dtype=tdt(dtype), device="cuda")
    out = torch.empty((B, 1024), dtype=torch.float32, device="cuda")

    def snapshot(kv):
        torch.cuda.synchronize()
        return out.cpu().numpy().copy(), to_bits(kv.k), to_bits(kv.v), kv.lens.cpu().numpy()

    kv_e, _ = paged_pair(101, lens, P, pps, dtype)
    base = kv_e.lens.clone()
    eager = []
    for r in range(3):
        ga.kv_crop([kv_e], base)
        x.copy_(xs[r])
        ga.layer_decode(cfg, L.dev, kv_e, x, out, ws)
        eager.append(snapshot(kv_e))
    kv_g, _ = paged_pair(101, lens, P, pps, dtype)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ga.layer_decode(cfg, L.dev, kv_g, x, out, ws)
    for r in range(3):
        ga.kv_crop([kv_g], base)
        x.copy_(xs[r])
        g.replay()
        got = snapshot(kv_g)
        assert all(np.array_equal(a, b) for a, b in zip(got, eager[r])), f"replay {r}"
        assert kv_g.status.item() == 0
    del g

    res = {}
    for entry in ("decode", "noalloc"):
        kv, _ = paged_pair(102, lens, P, pps, dtype)
        outs = []
        for rows in (B, 2):
            xb = to_dev(si.activations(102, 0, rows, rows, 1024, dtype), dtype)
            o = torch.empty((rows, 1024), dtype=torch.float32, device="cuda")
            st = _i32(list(range(rows))[::-1])
            if entry == "noalloc":
                ga.layer_decode_noalloc(cfg, L.dev, kv, xb, o, slots=st)
            else:
                ga.layer_decode(cfg, L.dev, kv, xb, o, ws, slots=st)
            torch.cuda.synchronize()
            outs.append(o.cpu().numpy())
        res[entry] = (outs, to_bits(kv.k), to_bits(kv.v), kv.lens.cpu().numpy(), kv.status.item())
    a, b = res["decode"], res["noalloc"]
    assert all(np.array_equal(p, q) for p, q in zip(a[0], b[0]))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])
    assert a[4] == b[4] == 0
