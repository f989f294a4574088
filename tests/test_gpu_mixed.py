"""GPU parity of mixed calls (decode rows and verify blocks of per-sequence sizes in one
dispatch) against the fp64 oracle, through the C ABI: every attention kernel that takes them
(equal-share waves for 2 and 4 q heads per kv head, the chunked kernel for 1 and 8), calls
of a few rows (which take the many-row kernels too), FP8 caches, multi-section rotary,
per-sequence overflow, the whole decoder layer, and blocks all of one size, which are the
decode or verify call itself."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import (TOL, SeededLayer, check_codes, check_rounded_rows, device_cache, device_cache_e4m3,
                        fill_cache, fill_cache_e4m3, oracle_cache, oracle_cache_e4m3, rel_err, tdt, to_bits,
                        to_dev)

pytestmark = pytest.mark.gpu


def _i32(v):
    return None if v is None else torch.tensor(np.asarray(v, np.int32).ravel(), dtype=torch.int32, device="cuda")


def _run_mixed(L, cfg, kv, xb, sizes, dtype, slots=None, positions=None, residual=None, host_lens=None):
    rows, H = xb.shape
    out = torch.empty((rows, H), dtype=torch.float32 if cfg.out_dtype == ga.F32 else tdt(dtype), device="cuda")
    ws = ga.alloc_workspace(cfg, rows, kv.c.capacity)
    ga.layer_mixed(cfg, L.dev, kv, to_dev(xb, dtype), sizes, out, ws, slots=_i32(slots), positions=_i32(positions),
                   residual=None if residual is None else to_dev(residual, dtype), host_lens=host_lens)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _run_verify(L, cfg, kv, xb, dtype, slots=None):
    B, k, H = xb.shape
    out = torch.empty((B, k, H), dtype=torch.float32, device="cuda")
    ws = ga.alloc_workspace(cfg, B * k, kv.c.capacity)
    ga.layer_verify(cfg, L.dev, kv, to_dev(xb, dtype), out, ws, slots=_i32(slots))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _run_decode(L, cfg, kv, xb, dtype, slots=None):
    B, H = xb.shape
    out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = ga.alloc_workspace(cfg, B, kv.c.capacity)
    ga.layer_decode(cfg, L.dev, kv, to_dev(xb, dtype), out, ws, slots=_i32(slots))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


CASES = {
    # name: (n_q_heads, n_kv_heads, block sizes, committed lengths)
    "few_rows": (16, 8, [1, 3], [40, 201]),
    "few_rows_3": (16, 8, [2, 1, 1], [0, 77, 255]),
    "waves_g2": (16, 8, [1, 4, 8, 1, 16, 2, 1], [30, 0, 250, 129, 7, 64, 283]),
    "waves_g4": (16, 4, [3, 1, 1, 7, 2], [100, 5, 260, 33, 1]),
    "chunked_g8": (16, 2, [5, 1, 2, 9], [12, 290, 0, 140]),
    "chunked_g1": (8, 8, [1, 2, 6, 1, 1], [61, 3, 199, 0, 240]),
    # more than 64 rows: several row tiles of the projections
    "waves_g2_rows140": (16, 8, [9, 1, 16, 4, 12, 7, 1, 16, 3, 10, 14, 2, 8, 16, 5, 16],
                         [150, 193, 236, 279, 0, 280, 231, 120, 100, 50, 283, 270, 17, 1, 90, 200]),
}


@pytest.mark.parametrize("dtype", [si.BF16, si.F16])
@pytest.mark.parametrize("case", sorted(CASES))
def test_mixed_vs_oracle(case, dtype):
    """Ragged block sizes with permuted slots, explicit positions and a residual: outputs, the
    appended cache rows (each within one unit of the oracle's rounding), untouched cache
    elsewhere, and every length advanced by its own block."""
    nq, nkv, sizes, lens = CASES[case]
    B, rows, cap = len(sizes), sum(sizes), 300
    seed = 50 + sorted(CASES).index(case)
    slots = list(range(B))[::-1]
    L = SeededLayer(seed, 0, 1024, dtype, nq=nq, nkv=nkv)
    kb, vb = fill_cache(seed, 0, lens, cap, dtype, nkv=nkv)
    xb = si.activations(seed, 0, 0, rows, 1024, dtype)
    res = si.residual(seed, 0, 0, rows, 1024, dtype)
    pos = [7 * b + 1000 * (b % 2) for b in range(B)]
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    ocfg = oracle.BlockConfig(hidden=1024, n_q_heads=nq, n_kv_heads=nkv, dtype=dtype)
    got = _run_mixed(L, ga.config(dtype=dtype, n_q_heads=nq, n_kv_heads=nkv), kv, xb, sizes, dtype, slots=slots,
                     positions=pos, residual=res, host_lens=[lens[s] for s in slots])
    want = oracle.mixed(ocfg, L.ref, ref, xb, sizes, slots=slots, positions=pos, residual_bits=res)
    err = rel_err(got, want)
    print(f"mixed {case} {dtype} sizes={sizes}: {err:.3e}")
    assert err < TOL[dtype]
    new = {s: lens[s] for s in range(B)}
    for b, s in enumerate(slots):
        new[s] += sizes[b]
    assert kv.lens.cpu().tolist() == [new[s] for s in range(B)] == ref.lens.tolist()
    assert kv.status.item() == 0
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    for b, s in enumerate(slots):
        l0, l1 = lens[s], lens[s] + sizes[b]
        check_rounded_rows(kg[s, :, l0:l1], ref.k[s, :, l0:l1], dtype)
        check_rounded_rows(vg[s, :, l0:l1], ref.v[s, :, l0:l1], dtype)
        assert np.array_equal(kg[s, :, :l0], kb[s, :, :l0]) and np.array_equal(kg[s, :, l1:], kb[s, :, l1:])
        assert np.array_equal(vg[s, :, :l0], vb[s, :, :l0]) and np.array_equal(vg[s, :, l1:], vb[s, :, l1:])


@pytest.mark.parametrize("B", [3, 10])
def test_mixed_blocks_of_one_row_are_the_decode_call_bit_for_bit(B):
    """Every block of one row: the decode call itself (same kernels, launch and bits)."""
    dtype = si.BF16
    lens = [5, 300, 0, 17, 129, 64, 250, 1, 33, 90][:B]
    L = SeededLayer(60, B, 1024, dtype)
    kb, vb = fill_cache(60, B, lens, 320, dtype)
    xb = si.activations(60, B, 0, B, 1024, dtype)
    cfg = ga.config(dtype=dtype)
    slots = list(range(B))[::-1]
    kv1, kv2 = device_cache(kb, vb, lens, dtype), device_cache(kb, vb, lens, dtype)
    a = _run_mixed(L, cfg, kv1, xb, [1] * B, dtype, slots=slots)
    d = _run_decode(L, cfg, kv2, xb, dtype, slots=slots)
    assert np.array_equal(a, d)
    assert torch.equal(kv1.k, kv2.k) and torch.equal(kv1.v, kv2.v) and torch.equal(kv1.lens, kv2.lens)


@pytest.mark.parametrize("nq,nkv,B,k", [(8, 8, 3, 4), (16, 8, 2, 2)])
def test_mixed_equal_blocks_are_the_verify_call_bit_for_bit(nq, nkv, B, k):
    """Blocks all of one size: the verify call with that k, bit for bit."""
    dtype = si.F16
    lens = [40, 0, 211][:B]
    L = SeededLayer(61, k, 1024, dtype, nq=nq, nkv=nkv)
    kb, vb = fill_cache(61, k, lens, 256, dtype, nkv=nkv)
    xb = si.activations(61, k, 0, B * k, 1024, dtype)
    cfg = ga.config(dtype=dtype, n_q_heads=nq, n_kv_heads=nkv)
    kv1, kv2 = device_cache(kb, vb, lens, dtype), device_cache(kb, vb, lens, dtype)
    a = _run_mixed(L, cfg, kv1, xb, [k] * B, dtype)
    v = _run_verify(L, cfg, kv2, xb.reshape(B, k, 1024), dtype).reshape(B * k, 1024)
    assert np.array_equal(a, v)
    assert torch.equal(kv1.k, kv2.k) and torch.equal(kv1.lens, kv2.lens)


def test_mixed_fp8_cache_vs_oracle_and_verify_bits():
    """FP8 cache on the equal-share attention: mixed blocks against the oracle (appended codes
    within one step), and equal blocks bit for bit with the verify entry point."""
    dtype = si.BF16
    sizes, lens = [1, 6, 2, 1, 8, 3], [300, 0, 45, 129, 7, 200]
    B, rows, cap = len(sizes), sum(sizes), 320
    L = SeededLayer(62, 0, 1024, dtype)
    kc, vc, ks, vs = fill_cache_e4m3(62, 0, lens, cap)
    xb = si.activations(62, 0, 0, rows, 1024, dtype)
    kv = device_cache_e4m3(kc, vc, lens, ks, vs)
    ref = oracle_cache_e4m3(kc, vc, lens, ks, vs)
    got = _run_mixed(L, ga.config(dtype=dtype), kv, xb, sizes, dtype)
    want = oracle.mixed(L.ocfg, L.ref, ref, xb, sizes)
    err = rel_err(got, want)
    print(f"mixed fp8 sizes={sizes}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + n for l, n in zip(lens, sizes)]
    kg = kv.k.cpu().numpy()
    for s in range(B):
        check_codes(kg[s, :, lens[s]:lens[s] + sizes[s]], ref.k[s, :, lens[s]:lens[s] + sizes[s]])
    # equal blocks: the verify call itself
    k = 4
    xb2 = si.activations(62, 1, 0, B * k, 1024, dtype)
    kv1, kv2 = device_cache_e4m3(kc, vc, lens, ks, vs), device_cache_e4m3(kc, vc, lens, ks, vs)
    a = _run_mixed(L, ga.config(dtype=dtype), kv1, xb2, [k] * B, dtype)
    v = _run_verify(L, ga.config(dtype=dtype), kv2, xb2.reshape(B, k, 1024), dtype).reshape(B * k, 1024)
    assert np.array_equal(a, v)
    assert torch.equal(kv1.k, kv2.k) and torch.equal(kv1.v, kv2.v)


@pytest.mark.parametrize("sizes", [[1, 3], [2, 1, 5, 1, 4]])
def test_mixed_multi_section_rotary_vs_oracle(sizes):
    dtype = si.BF16
    sections = (16, 24, 24)
    B, rows = len(sizes), sum(sizes)
    lens = [30, 250, 3, 77, 129][:B]
    L = SeededLayer(63, B, 1024, dtype)
    ocfg = oracle.BlockConfig(hidden=1024, dtype=dtype, mrope_sections=sections)
    kb, vb = fill_cache(63, B, lens, 300, dtype)
    pos3 = np.array([[100, 7, 2000, 5, 64][:B], [3, 900, 11, 70, 1][:B], [4000, 50, 9, 8, 300][:B]], np.int32)
    xb = si.activations(63, B, 0, rows, 1024, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    got = _run_mixed(L, ga.config(dtype=dtype, mrope_sections=sections), kv, xb, sizes, dtype, positions=pos3)
    want = oracle.mixed(ocfg, L.ref, ref, xb, sizes, positions=pos3)
    err = rel_err(got, want)
    print(f"mixed mrope sizes={sizes}: {err:.3e}")
    assert err < TOL[dtype]


@pytest.mark.parametrize("sizes,over", [([2, 2], 1), ([1, 5, 3, 1], 2)])
def test_mixed_overflow_of_one_sequence(sizes, over):
    """Sequence `over` would pass the capacity: its rows are NaN, its length and cache rows stay,
    the capacity bit is set; the other sequences are still right."""
    dtype = si.F16
    cap = 200
    lens = [10, 150, 60, 199][:len(sizes)]
    lens[over] = cap - sizes[over] + 1
    B, rows = len(sizes), sum(sizes)
    L = SeededLayer(64, B, 1024, dtype)
    kb, vb = fill_cache(64, B, lens, cap, dtype)
    xb = si.activations(64, B, 0, rows, 1024, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    got = _run_mixed(L, ga.config(dtype=dtype), kv, xb, sizes, dtype)
    want = oracle.mixed(L.ocfg, L.ref, ref, xb, sizes)
    r0 = sum(sizes[:over])
    bad = np.zeros(rows, bool)
    bad[r0:r0 + sizes[over]] = True
    assert np.all(np.isnan(got[bad])) and np.all(np.isfinite(got[~bad]))
    err = rel_err(got[~bad], want[~bad])
    print(f"mixed overflow sizes={sizes}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.status.item() == ga.STATUS_CAPACITY == ref.status
    assert kv.lens.cpu().tolist() == [l + (0 if b == over else n) for b, (l, n) in enumerate(zip(lens, sizes))]
    assert np.array_equal(to_bits(kv.k)[over], kb[over])


def test_decoder_layer_mixed_vs_oracle():
    from test_gpu_mlp import SeededMlp
    dtype = si.BF16
    sizes, lens = [1, 4, 1, 8, 2], [795, 0, 17, 300, 64]
    B, rows, cap = len(sizes), sum(sizes), 810
    L = SeededLayer(65, 0, 1024, dtype)
    M = SeededMlp(65, 0, 1024, 3072, dtype)
    kb, vb = fill_cache(65, 0, lens, cap, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = si.activations(65, 0, 0, rows, 1024, dtype)
    acfg, mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype)
    out = torch.empty((rows, 1024), dtype=torch.float32, device="cuda")
    ws = ga.decoder_layer_workspace(acfg, mcfg, rows, cap)
    ga.decoder_layer_mixed(acfg, L.dev, mcfg, M.dev, kv, to_dev(xb, dtype), sizes, out, ws, host_lens=lens)
    torch.cuda.synchronize()
    want = oracle.decoder_layer_mixed(L.ocfg, L.ref, M.ocfg, M.ref, ref, xb, sizes)
    err = rel_err(out.cpu().numpy(), want)
    print(f"decoder layer mixed sizes={sizes}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + n for l, n in zip(lens, sizes)]
