"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Small and mid-size cases that span several split-KV chunks with ragged tails,
every dtype, verify block sizes, crop and append, error paths on the device.
"""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import (TOL, SeededLayer, device_cache, fill_cache, oracle_cache, rel_err, tdt, to_bits,
                        to_dev, check_rounded_rows)

pytestmark = pytest.mark.gpu


def _x(stream, layer, step, shape, dtype):
    rows = int(np.prod(shape[:-1]))
    return si.activations(stream, layer, step, rows, shape[-1], dtype).reshape(shape)


# Agreement of two dispatch modes: the same fp32 arithmetic summed in a different order
# (wave shapes, where the chunk partials are merged).
AGREE = 1e-5


def _run_decode(L, cfg, kv, xb, dtype, slots=None, positions=None, residual=None, host_lens=None, ws=None):
    B, H = xb.shape
    out = torch.empty((B, H), dtype=torch.float32 if cfg.out_dtype == ga.F32 else tdt(dtype), device="cuda")
    ws = ga.alloc_workspace(cfg, B, kv.c.capacity) if ws is None else ws
    ga.layer_decode(cfg, L.dev, kv, to_dev(xb, dtype), out, ws,
                    slots=None if slots is None else torch.tensor(slots, dtype=torch.int32, device="cuda"),
                    positions=None if positions is None else torch.tensor(positions, dtype=torch.int32, device="cuda"),
                    residual=None if residual is None else to_dev(residual, dtype), host_lens=host_lens)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dispatch", [0, 1, 2])
def test_single_layer_decode_bs1_kv64(dispatch):
    """Single layer, bs1, fp16, hidden 1024, KV 64, new token at position 64."""
    dtype, cap = si.F16, 128
    L = SeededLayer(1, 0, 1024, dtype)
    kb, vb = fill_cache(1, 0, [64], cap, dtype)
    kv = device_cache(kb, vb, [64], dtype)
    ref = oracle_cache(kb, vb, [64], dtype)
    xb = _x(1, 0, 0, (1, 1024), dtype)
    got = _run_decode(L, ga.config(dtype="f16", dispatch=dispatch), kv, xb, dtype)
    want = oracle.decode(L.ocfg, L.ref, ref, xb)
    err = rel_err(got, want)
    print(f"single layer bs1 dispatch={dispatch} max|err|/rms = {err:.3e}")
    assert err < TOL[dtype]
    assert int(kv.lens.item()) == 65 and int(kv.status.item()) == 0
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    check_rounded_rows(kg[0, :, 64], ref.k[0, :, 64], dtype)
    check_rounded_rows(vg[0, :, 64], ref.v[0, :, 64], dtype)
    untouched = np.ones(kg.shape, bool)
    untouched[0, :, 64] = False
    assert np.array_equal(kg[untouched], kb[untouched]) and np.array_equal(vg[untouched], vb[untouched])


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("split", [0, 16, 48, 1024])
@pytest.mark.parametrize("dispatch", [0, 1])
def test_ragged_decode_vs_oracle(dtype, split, dispatch):
    lens = [0, 1, 17, 100, 333, 64]
    cap = 400
    slots = [3, 0, 5, 4, 1, 2]
    L = SeededLayer(2, 1, 1024, dtype)
    kb, vb = fill_cache(2, 1, lens, cap, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = _x(2, 1, 3, (6, 1024), dtype)
    got = _run_decode(L, ga.config(dtype=dtype, kv_split=split, dispatch=dispatch), kv, xb, dtype, slots=slots)
    want = oracle.decode(L.ocfg, L.ref, ref, xb, slots=slots)
    err = rel_err(got, want)
    print(f"ragged {dtype} split={split} dispatch={dispatch}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + 1 for l in lens]
    kg = to_bits(kv.k)
    for s in range(6):
        check_rounded_rows(kg[s, :, lens[s]], ref.k[s, :, lens[s]], dtype)


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("split", [0, 32, 512])
def test_few_rows_stale_host_lengths(dtype, split):
    """Up to 4 rows, the host's copy of the lengths far below the device's: the launch is sized
    for fewer chunks than the rows have, so workgroups take several chunks each and the o_proj
    merge reads past its first batch of partials; chunks of 512 keys take steps past the loaded
    ones.  Results follow the device lengths (the truth), decode and verify."""
    lens = [700, 33, 250]
    host = [100, 10, 20]
    cap = 800
    L = SeededLayer(2, 3, 1024, dtype)
    kb, vb = fill_cache(2, 3, lens, cap, dtype)
    cfg = ga.config(dtype=dtype, kv_split=split)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = _x(2, 3, 0, (3, 1024), dtype)
    got = _run_decode(L, cfg, kv, xb, dtype, host_lens=host)
    want = oracle.decode(L.ocfg, L.ref, ref, xb)
    err = rel_err(got, want)
    print(f"stale host lens decode {dtype} split={split}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + 1 for l in lens]
    kg = to_bits(kv.k)
    for s in range(3):
        check_rounded_rows(kg[s, :, lens[s]], ref.k[s, :, lens[s]], dtype)
    # verify: 2 sequences x 2 rows, host copy stale
    kv2 = device_cache(kb[:2], vb[:2], lens[:2], dtype)
    ref2 = oracle_cache(kb[:2], vb[:2], lens[:2], dtype)
    xv = _x(2, 3, 1, (2, 2, 1024), dtype)
    out = torch.empty((2, 2, 1024), dtype=torch.float32, device="cuda")
    ws = ga.alloc_workspace(cfg, 4, cap)
    ga.layer_verify(cfg, L.dev, kv2, to_dev(xv, dtype), out, ws, host_lens=host[:2])
    torch.cuda.synchronize()
    gotv = out.cpu().numpy().astype(np.float64)
    wantv = oracle.verify(L.ocfg, L.ref, ref2, xv)
    errv = rel_err(gotv, wantv)
    print(f"stale host lens verify {dtype} split={split}: {errv:.3e}")
    assert errv < TOL[dtype]
    assert kv2.lens.cpu().tolist() == [l + 2 for l in lens[:2]]


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("B", [2, 6])
def test_positions_residual_and_16bit_out(dtype, B):
    """Explicit positions, a residual and 16-bit output; B = 6 takes the many-row kernels."""
    lens = [10, 250, 0, 77, 1, 299][:B]
    L = SeededLayer(2, 2, 2048, dtype)
    kb, vb = fill_cache(2, 2, lens, 300, dtype)
    xb = _x(2, 2, 0, (B, 2048), dtype)
    res = si.residual(2, 2, 0, B, 2048, dtype)
    pos = [1000, 3, 0, 77, 4095, 12][:B]
    for out_dt in ("f32", dtype):
        kv = device_cache(kb, vb, lens, dtype)
        ref = oracle_cache(kb, vb, lens, dtype)
        got = _run_decode(L, ga.config(hidden=2048, dtype=dtype, out_dtype=out_dt), kv, xb, dtype,
                          positions=pos, residual=res, host_lens=lens)
        want = oracle.decode(L.ocfg, L.ref, ref, xb, positions=pos, residual_bits=res)
        err = rel_err(got, want)
        print(f"pos/res {dtype} out={out_dt}: {err:.3e}")
        if out_dt == "f32":
            assert err < TOL[dtype]
        else:   # a 16-bit output: each value within one unit in the last place of the rounded
            # oracle value, or within OUT16_REL times the output RMS of it
            frac = check_rounded_rows(oracle.rne16(got, dtype), oracle.rne16(want, dtype), dtype, rel=OUT16_REL)
            print(f"  16-bit out: {frac:.3%} of the values differ from the rounded oracle")


def test_group_sizes_and_shapes():
    """q heads per kv head 1, 2, 4, 8 (the index map i // group) at hidden 512 and 1536."""
    dtype = si.F16
    for hidden, nq, nkv in [(512, 4, 4), (1536, 8, 4), (1024, 16, 4), (1024, 16, 2)]:
        L = SeededLayer(9, nq * 10 + nkv, hidden, dtype, nq=nq, nkv=nkv)
        lens = [7, 130]
        kb, vb = fill_cache(9, nq, lens, 160, dtype, nkv=nkv)
        kv = device_cache(kb, vb, lens, dtype)
        ref = oracle_cache(kb, vb, lens, dtype)
        xb = _x(9, nq, 0, (2, hidden), dtype)
        got = _run_decode(L, ga.config(hidden=hidden, n_q_heads=nq, n_kv_heads=nkv), kv, xb, dtype)
        want = oracle.decode(L.ocfg, L.ref, ref, xb)
        err = rel_err(got, want)
        print(f"H={hidden} nq={nq} nkv={nkv}: {err:.3e}")
        assert err < TOL[dtype]


def test_many_row_group_sizes():
    """Six rows (matrix-core projections, many-row attention for groups 2 and 4, the
    chunked attention for groups 1 and 8) against the oracle."""
    dtype = si.BF16
    lens = [7, 130, 0, 64, 250, 1]
    for hidden, nq, nkv in [(1024, 16, 4), (1024, 16, 8), (512, 4, 4), (1024, 16, 2)]:
        L = SeededLayer(9, nq * 10 + nkv + 1, hidden, dtype, nq=nq, nkv=nkv)
        kb, vb = fill_cache(9, nq + 1, lens, 260, dtype, nkv=nkv)
        xb = _x(9, nq + 1, 0, (len(lens), hidden), dtype)
        for split in (0, 16):
            kvr = device_cache(kb, vb, lens, dtype)
            got = _run_decode(L, ga.config(hidden=hidden, n_q_heads=nq, n_kv_heads=nkv, dtype=dtype, kv_split=split),
                              kvr, xb, dtype)
            ref = oracle_cache(kb, vb, lens, dtype)
            want = oracle.decode(L.ocfg, L.ref, ref, xb)
            err = rel_err(got, want)
            print(f"6 rows H={hidden} nq={nq} nkv={nkv} split={split}: {err:.3e}")
            assert err < TOL[dtype]
            assert kvr.lens.cpu().tolist() == [l + 1 for l in lens]
            kg = to_bits(kvr.k)
            for s in range(len(lens)):
                check_rounded_rows(kg[s, :, lens[s]], ref.k[s, :, lens[s]], dtype)


def test_many_row_device_side_errors():
    """Six rows, two of them past the capacity and one in a slot outside the cache: those
    rows are NaN, their lengths stay, the status word says why; the others are right."""
    dtype = si.BF16
    lens = [16, 5, 16, 0, 9, 3]
    L = SeededLayer(4, 1, 1024, dtype)
    kb, vb = fill_cache(4, 1, lens, 16, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    xb = _x(4, 1, 0, (6, 1024), dtype)
    got = _run_decode(L, ga.config(dtype=dtype), kv, xb, dtype)
    bad = [0, 2]
    for r in range(6):
        assert np.all(np.isnan(got[r])) if r in bad else np.all(np.isfinite(got[r]))
    assert kv.lens.cpu().tolist() == [16, 6, 16, 1, 10, 4] and kv.status.item() == ga.STATUS_CAPACITY
    good = [r for r in range(6) if r not in bad]
    sub = [lens[r] for r in good]
    want = oracle.decode(L.ocfg, L.ref, oracle_cache(kb[good], vb[good], sub, dtype), xb[good])
    assert rel_err(got[good], want) < TOL[dtype]
    kv2 = device_cache(kb, vb, lens, dtype)
    got = _run_decode(L, ga.config(dtype=dtype), kv2, xb[:5], dtype, slots=[1, 3, 9, 4, 5])
    assert np.all(np.isnan(got[2])) and all(np.all(np.isfinite(got[r])) for r in (0, 1, 3, 4))
    assert kv2.status.item() == ga.STATUS_BAD_SLOT
    assert kv2.lens.cpu().tolist() == [16, 6, 16, 1, 10, 4]


def test_determinism_and_split_invariance():
    dtype = si.BF16
    lens = [900, 37, 512]
    L = SeededLayer(3, 0, 1024, dtype)
    kb, vb = fill_cache(3, 0, lens, 1024, dtype)
    xb = _x(3, 0, 0, (3, 1024), dtype)
    outs = {}
    for split, rep in [(16, 0), (16, 1), (64, 0), (256, 0)]:
        kv = device_cache(kb, vb, lens, dtype)
        outs[(split, rep)] = _run_decode(L, ga.config(dtype=dtype, kv_split=split), kv, xb, dtype)
    assert np.array_equal(outs[(16, 0)], outs[(16, 1)])
    for split in (64, 256):
        assert rel_err(outs[(split, 0)], outs[(16, 0)]) < 1e-4


def _run_verify(L, cfg, kv, xb, dtype, slots=None, positions=None, ws=None, residual=None, host_lens=None):
    B, k, H = xb.shape
    out = torch.empty((B, k, H), dtype=torch.float32 if cfg.out_dtype == ga.F32 else tdt(dtype), device="cuda")
    ws = ga.alloc_workspace(cfg, B * k, kv.c.capacity) if ws is None else ws
    ga.layer_verify(cfg, L.dev, kv, to_dev(xb, dtype), out, ws,
                    slots=None if slots is None else torch.tensor(slots, dtype=torch.int32, device="cuda"),
                    positions=None if positions is None else torch.tensor(positions, dtype=torch.int32, device="cuda"),
                    residual=None if residual is None else to_dev(residual, dtype), host_lens=host_lens)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# A 16-bit output is the kernel's fp32 result rounded once: each value within one unit in the
# last place of the rounded oracle value (the two can straddle a rounding boundary), or within
# this fraction of the output RMS of it (near zero, where a unit is tiny).  The fp32 results
# sit about 1e-6 (vector path) to 1.2e-5 (two-term matrix-core path) of the RMS from the oracle.
OUT16_REL = 5e-5


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("B,k,over", [(1, 4, None), (2, 2, 0), (3, 8, 1), (2, 16, None)])
def test_verify_positions_residual_16bit_out_and_overflow(dtype, B, k, over):
    """Verify with explicit per-sequence positions (row r turns by positions[b] + r), a [B][k][H]
    residual, fp32 and 16-bit outputs, on the few-row kernels (B k <= 4) and the matrix-core path
    (B k > 4).  Sequence `over` would pass the capacity: its k rows are NaN, its length and cache
    rows stay and the capacity bit is set, while the other sequences are still right.  `over`
    names the overflowing slot; sequences map to slots in reverse order."""
    cap = 300
    lens = [40, 201, 7][:B]
    if over is not None:
        lens[over] = cap - k + 1
    slots = list(range(B))[::-1]
    H = 1024 if k != 16 else 2048
    L = SeededLayer(7, 10 * B + k, H, dtype)
    kb, vb = fill_cache(7, 10 * B + k, lens, cap, dtype)
    xb = _x(7, 10 * B + k, 0, (B, k, H), dtype)
    res = si.residual(7, 10 * B + k, 0, B * k, H, dtype).reshape(B, k, H)
    pos = [4000, 12, 777][:B]
    ok = [b for b in range(B) if slots[b] != over]
    for out_dt in ("f32", dtype):
        kv = device_cache(kb, vb, lens, dtype)
        ref = oracle_cache(kb, vb, lens, dtype)
        got = _run_verify(L, ga.config(hidden=H, dtype=dtype, out_dtype=out_dt), kv, xb, dtype, slots=slots,
                          positions=pos, residual=res)
        # the oracle's cache slot s holds sequence slots.index(s); lens given per slot
        want = oracle.verify(L.ocfg, L.ref, ref, xb, slots=slots, positions=pos, residual_bits=res)
        for b in range(B):
            assert np.all(np.isnan(got[b])) if slots[b] == over else np.all(np.isfinite(got[b])), b
        if out_dt == "f32":
            err = rel_err(got[ok], want[ok])
            print(f"verify B={B} k={k} {dtype} pos/res f32: {err:.3e}")
            assert err < TOL[dtype]
        else:
            frac = check_rounded_rows(oracle.rne16(got[ok], dtype), oracle.rne16(want[ok], dtype), dtype,
                                      rel=OUT16_REL)
            print(f"verify B={B} k={k} {dtype} pos/res 16-bit: {frac:.3%} differ from the rounded oracle")
        assert kv.lens.cpu().tolist() == [lens[s] + (0 if s == over else k) for s in range(B)]
        assert kv.status.item() == (0 if over is None else ga.STATUS_CAPACITY) == ref.status
        kg, vg = to_bits(kv.k), to_bits(kv.v)
        for b in range(B):
            s = slots[b]
            if s == over:
                assert np.array_equal(kg[s], kb[s]) and np.array_equal(vg[s], vb[s])
            else:
                l0 = lens[s]
                check_rounded_rows(kg[s, :, l0:l0 + k], ref.k[s, :, l0:l0 + k], dtype)
                check_rounded_rows(vg[s, :, l0:l0 + k], ref.v[s, :, l0:l0 + k], dtype)


@pytest.mark.parametrize("k", [1, 3, 8, 16, 32])
@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
def test_verify_vs_oracle(k, dtype):
    lens = [5, 64, 200]
    slots = [2, 0, 1]
    L = SeededLayer(3, 1, 1024, dtype)
    kb, vb = fill_cache(3, 1, lens, 256, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = _x(3, 1, k, (3, k, 1024), dtype)
    got = _run_verify(L, ga.config(dtype=dtype), kv, xb, dtype, slots=slots)
    want = oracle.verify(L.ocfg, L.ref, ref, xb, slots=slots)
    err = rel_err(got, want)
    print(f"verify k={k} {dtype}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + k for l in lens]
    kg = to_bits(kv.k)
    for b, s in enumerate(slots):
        check_rounded_rows(kg[s, :, lens[s]:lens[s] + k], ref.k[s, :, lens[s]:lens[s] + k], dtype)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_verify_rows_equal_sequential_decode_rows(k):
    """Verify rows agree with k single-token steps: bit for bit when both calls take the
    same projection path (up to 4 rows: vector ALU) and chunking, else to rounding."""
    dtype = si.F16
    lens = [795]
    L = SeededLayer(3, 2, 1024, dtype)
    kb, vb = fill_cache(3, 2, lens, 832, dtype)
    xb = _x(3, 2, 0, (1, k, 1024), dtype)
    cfg = ga.config(dtype=dtype, kv_split=32)
    kv1 = device_cache(kb, vb, lens, dtype)
    ov = _run_verify(L, cfg, kv1, xb, dtype)
    kv2 = device_cache(kb, vb, lens, dtype)
    od = np.stack([_run_decode(L, cfg, kv2, xb[:, r, :], dtype) for r in range(k)], axis=1)
    if k <= 4:
        assert np.array_equal(ov, od)
        assert np.array_equal(to_bits(kv1.k), to_bits(kv2.k)) and np.array_equal(to_bits(kv1.v), to_bits(kv2.v))
    else:
        assert rel_err(ov, od) < 1e-5
    # the automatic chunking may differ between the two; then they agree to rounding
    kv3 = device_cache(kb, vb, lens, dtype)
    ov3 = _run_verify(L, ga.config(dtype=dtype), kv3, xb, dtype)
    assert rel_err(ov3, od) < 1e-4


@pytest.mark.parametrize("a", [0, 1, 5, 8])
def test_crop_after_rejection_equals_never_appended(a):
    """Verify k = 8, crop to the accepted prefix a, poison the dropped rows with NaN: the
    next decode is bit-identical to a cache that only ever received the accepted rows
    (copied bit for bit from the verify call) and no rejected one."""
    dtype, k = si.F16, 8
    lens = [795]
    L = SeededLayer(3, 3, 1024, dtype)
    kb, vb = fill_cache(3, 3, lens, 832, dtype)
    xs = _x(3, 3, 1, (1, k, 1024), dtype)
    xn = _x(3, 3, 2, (1, 1024), dtype)
    cfg = ga.config(dtype=dtype, kv_split=64)
    spec = device_cache(kb, vb, lens, dtype)
    _run_verify(L, cfg, spec, xs, dtype)
    ga.kv_crop([spec], torch.tensor([795 + a], dtype=torch.int32, device="cuda"))
    accepted_k = spec.k[0, :, 795:795 + a].clone()
    accepted_v = spec.v[0, :, 795:795 + a].clone()
    spec.k[0, :, 795 + a:] = float("nan")
    spec.v[0, :, 795 + a:] = float("nan")
    ref = device_cache(kb, vb, [795 + a], dtype)
    ref.k[0, :, 795:795 + a] = accepted_k
    ref.v[0, :, 795:795 + a] = accepted_v
    o_spec = _run_decode(L, cfg, spec, xn, dtype)
    o_ref = _run_decode(L, cfg, ref, xn, dtype)
    assert np.all(np.isfinite(o_spec))
    assert np.array_equal(o_spec, o_ref)
    assert spec.lens.item() == ref.lens.item() == 795 + a + 1 and spec.status.item() == 0


def test_kv_append_and_crop_bit_exact():
    dtype = si.BF16
    cap, nkv = 40, 8
    lens0 = np.array([3, 0, 10, 38], np.int32)
    g = np.random.default_rng(5)
    kb = g.integers(0, 2 ** 16, (4, nkv, cap, 128)).astype(np.uint16)
    vb = g.integers(0, 2 ** 16, (4, nkv, cap, 128)).astype(np.uint16)
    layers = [device_cache(kb, vb, lens0, dtype) for _ in range(3)]
    kn = g.integers(0, 2 ** 16, (3, 5, nkv, 128)).astype(np.uint16)
    vn = g.integers(0, 2 ** 16, (3, 5, nkv, 128)).astype(np.uint16)
    slots = [2, 0, 3]                      # slot 3 (length 38) overflows capacity 40 with 5 rows
    ga.kv_append(layers[0], to_dev(kn, dtype), to_dev(vn, dtype),
                 slots=torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.KVCache(kb.copy(), vb.copy(), lens0.astype(np.int64), dtype)
    oracle.kv_append(ref, kn, vn, slots=slots)
    assert np.array_equal(to_bits(layers[0].k), ref.k) and np.array_equal(to_bits(layers[0].v), ref.v)
    assert layers[0].lens.cpu().tolist() == ref.lens.tolist() == [8, 0, 15, 38]
    assert layers[0].status.item() == ga.STATUS_CAPACITY == ref.status
    # crop all three layers in one call; layer 0 grew, the others still have lens0
    new = torch.tensor([2, 0, 12, 38], dtype=torch.int32, device="cuda")
    ga.kv_crop(layers, new)
    torch.cuda.synchronize()
    assert layers[0].lens.cpu().tolist() == [2, 0, 12, 38]
    assert layers[1].lens.cpu().tolist() == [2, 0, 10, 38] and layers[1].status.item() == ga.STATUS_CROP_GROW
    assert np.array_equal(to_bits(layers[0].k), ref.k)          # crop never touches data


def test_device_side_errors_write_nan_and_set_status():
    dtype = si.F16
    lens = [16, 5, 16]
    L = SeededLayer(4, 0, 1024, dtype)
    kb, vb = fill_cache(4, 0, lens, 16, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    xb = _x(4, 0, 0, (3, 1024), dtype)
    got = _run_decode(L, ga.config(dtype=dtype), kv, xb, dtype)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[2])) and np.all(np.isfinite(got[1]))
    assert kv.lens.cpu().tolist() == [16, 6, 16] and kv.status.item() == ga.STATUS_CAPACITY
    # a slot outside [0, batch_cap)
    kv2 = device_cache(kb, vb, lens, dtype)
    got = _run_decode(L, ga.config(dtype=dtype), kv2, xb[:2], dtype, slots=[1, 7])
    assert np.all(np.isfinite(got[0])) and np.all(np.isnan(got[1]))
    assert kv2.status.item() == ga.STATUS_BAD_SLOT


def test_host_side_validation():
    dtype = si.F16
    L = SeededLayer(4, 1, 1024, dtype)
    kb, vb = fill_cache(4, 1, [4], 8, dtype)
    kv = device_cache(kb, vb, [4], dtype)
    x = to_dev(_x(4, 1, 0, (1, 1024), dtype), dtype)
    out = torch.empty((1, 1024), dtype=torch.float32, device="cuda")
    cfg = ga.config()
    ws = ga.alloc_workspace(cfg, 1, 8)
    with pytest.raises(ga.AsrError) as e:
        ga.layer_decode(cfg, L.dev, kv, x, out, ws, host_lens=[8])
    assert e.value.code == -3
    with pytest.raises(ga.AsrError) as e:
        ga.layer_decode(cfg, L.dev, kv, x, out, ws[:100])
    assert e.value.code == -4
    with pytest.raises(ga.AsrError) as e:
        ga.layer_decode(ga.config(head_dim=64), L.dev, kv, x, out, ws)
    assert e.value.code == -2
    assert kv.lens.item() == 4     # nothing was enqueued


@pytest.mark.parametrize("case", ["decode_bs1", "decode_ragged", "verify"])
def test_fused_and_stream_ordered_dispatch_agree(case):
    """The fused single-dispatch kernel and the three stream-ordered kernels compute the same
    softmax sums in a different order (wave shapes, where the chunks are merged): fp32 outputs
    within AGREE of their RMS of each other; identical cache bits and lengths."""
    dtype = si.F16 if case != "decode_ragged" else si.BF16
    lens = {"decode_bs1": [795], "decode_ragged": [3, 700, 1200, 0], "verify": [795]}[case]
    cap = 1280
    L = SeededLayer(5, 1, 1024, dtype)
    kb, vb = fill_cache(5, 1, lens, cap, dtype)
    res = {}
    for mode in (ga.DISPATCH_MULTI, ga.DISPATCH_FUSED):
        kv = device_cache(kb, vb, lens, dtype)
        cfg = ga.config(dtype=dtype, dispatch=mode)
        if case == "verify":
            out = _run_verify(L, cfg, kv, _x(5, 1, 0, (len(lens), 4, 1024), dtype), dtype)
        else:
            out = _run_decode(L, cfg, kv, _x(5, 1, 0, (len(lens), 1024), dtype), dtype)
        res[mode] = (out, to_bits(kv.k), to_bits(kv.v), kv.lens.cpu().numpy(), kv.status.item())
    a, b = res[ga.DISPATCH_MULTI], res[ga.DISPATCH_FUSED]
    assert np.max(np.abs(a[0] - b[0])) <= AGREE * np.sqrt(np.mean(a[0] ** 2))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert np.array_equal(a[3], b[3]) and a[4] == b[4] == 0


def test_fused_dispatch_rejects_shapes_without_an_instance():
    """The fused dispatch exists for the pages' shapes and up to 4 rows only."""
    dtype = si.F16
    L2 = SeededLayer(5, 2, 1024, dtype)
    kb2, vb2 = fill_cache(5, 2, [10] * 5, 32, dtype)
    kv2 = device_cache(kb2, vb2, [10] * 5, dtype)
    cfg_fused = ga.config(dispatch=ga.DISPATCH_FUSED)
    with pytest.raises(ga.AsrError) as e:
        ga.layer_decode(cfg_fused, L2.dev, kv2, to_dev(_x(5, 2, 0, (5, 1024), dtype), dtype),
                        torch.empty((5, 1024), dtype=torch.float32, device="cuda"), ga.alloc_workspace(cfg_fused, 5, 32))
    assert e.value.code == -2
    L = SeededLayer(9, 44, 512, dtype, nq=4, nkv=4)
    kb, vb = fill_cache(9, 4, [3], 16, dtype, nkv=4)
    kv = device_cache(kb, vb, [3], dtype)
    cfg = ga.config(hidden=512, n_q_heads=4, n_kv_heads=4, dispatch=ga.DISPATCH_FUSED)
    out = torch.empty((1, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(ga.AsrError) as e:
        ga.layer_decode(cfg, L.dev, kv, to_dev(_x(9, 4, 0, (1, 512), dtype), dtype), out,
                        ga.alloc_workspace(cfg, 1, 16))
    assert e.value.code == -2


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("rows", [5, 16, 64, 65, 130])
def test_matrix_core_projections_vs_oracle(dtype, rows):
    """More than 4 rows run the projections on MFMA (two-term split of fp32 operands),
    including ragged row counts that leave partial 16-row and 64-row blocks."""
    lens = [int(v) for v in np.random.default_rng(rows).integers(0, 300, rows)]
    H = 2048 if rows == 65 else 1024
    L = SeededLayer(6, rows, H, dtype)
    kb, vb = fill_cache(6, rows, lens, 320, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    pick = sorted({0, rows - 1, rows // 2, 3})
    ref = oracle_cache(kb, vb, lens, dtype, seqs=pick)
    xb = _x(6, rows, 0, (rows, H), dtype)
    res = si.residual(6, rows, 0, rows, H, dtype)
    got = _run_decode(L, ga.config(hidden=H, dtype=dtype), kv, xb, dtype, residual=res)
    want = oracle.decode(L.ocfg, L.ref, ref, xb[pick], residual_bits=res[pick])
    err = rel_err(got[pick], want)
    print(f"mfma rows={rows} H={H} {dtype}: {err:.3e}")
    assert err < TOL[dtype]
    kg = to_bits(kv.k)
    for i, sq in enumerate(pick):
        check_rounded_rows(kg[sq, :, lens[sq]], ref.k[i, :, lens[sq]], dtype)


@pytest.mark.parametrize("rows", [1, 64])
def test_phase_events_leave_results_unchanged(rows):
    """Launching the phase kernels with diagnostics events (hipExtLaunchKernelGGL) computes the
    same bits as the plain launch, and stamps three positive, ordered kernel durations."""
    dtype = si.BF16
    lens = si.kv_lengths(4, rows, 200, 1500).tolist()
    L = SeededLayer(4, 3, 1024, dtype)
    kb, vb = fill_cache(4, 3, lens, 1536, dtype)
    x = _x(4, 3, 0, (rows, 1024), dtype)
    res = []
    for with_events in (False, True):
        kv = device_cache(kb, vb, lens, dtype)
        cfg = ga.config(dtype=dtype, dispatch=ga.DISPATCH_MULTI)
        pe = ga.PhaseEvents()
        if with_events:
            cfg.phase_events = pe.ptr
        res.append((_run_decode(L, cfg, kv, x, dtype), to_bits(kv.k), kv.lens.cpu().numpy()))
        if with_events:
            torch.cuda.synchronize()
            d = pe.elapsed_ms()
            assert all(0.0 < t < 50.0 for t in d), d
            assert pe.total_ms() >= sum(d) * 0.999
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1]) and np.array_equal(res[0][2], res[1][2])


@pytest.mark.parametrize("case", ["bs1", "rows3_with_overflow", "verify2x2"])
def test_fused_dispatch_reuses_its_workspace(case):
    """Several one-dispatch calls in a row on one workspace (its counters must return to zero
    after every call) agree with the stream-ordered kernels (fp32 outputs within AGREE of their
    RMS, NaN in the same places; cache bits, lengths and status identical), including rows whose
    append overflows the capacity (NaN out, length kept, status bit)."""
    dtype = si.F16 if case != "verify2x2" else si.BF16
    lens = {"bs1": [300], "rows3_with_overflow": [40, 64, 7], "verify2x2": [100, 33]}[case]
    n = 2 if case == "verify2x2" else 1
    cap = {"bs1": 320, "rows3_with_overflow": 64, "verify2x2": 128}[case]
    L = SeededLayer(6, 2, 1024, dtype)
    kb, vb = fill_cache(6, 2, lens, cap, dtype)
    res = {}
    for mode in (ga.DISPATCH_MULTI, ga.DISPATCH_FUSED):
        kv = device_cache(kb, vb, lens, dtype)
        cfg = ga.config(dtype=dtype, dispatch=mode, kv_split=32)
        ws = ga.alloc_workspace(cfg, len(lens) * n, cap)
        outs = []
        for step in range(3):
            if n == 1:
                outs.append(_run_decode(L, cfg, kv, _x(6, 2, step, (len(lens), 1024), dtype), dtype, ws=ws))
            else:
                outs.append(_run_verify(L, cfg, kv, _x(6, 2, step, (len(lens), n, 1024), dtype), dtype, ws=ws))
        res[mode] = (outs, to_bits(kv.k), to_bits(kv.v), kv.lens.cpu().numpy(), kv.status.item())
    a, b = res[ga.DISPATCH_MULTI], res[ga.DISPATCH_FUSED]
    for oa, ob in zip(a[0], b[0]):
        assert np.array_equal(np.isnan(oa), np.isnan(ob))
        fa, fb = oa[~np.isnan(oa)], ob[~np.isnan(ob)]
        assert np.max(np.abs(fa - fb)) <= AGREE * np.sqrt(np.mean(fa ** 2))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    assert np.array_equal(a[3], b[3]) and a[4] == b[4]
    if case == "rows3_with_overflow":
        assert b[4] == ga.STATUS_CAPACITY and np.all(np.isnan(b[0][0][1])) and b[3][1] == 64
    else:
        assert b[4] == 0


def test_fused_dispatch_workspace_across_changing_shapes():
    """One workspace serves one-dispatch calls of 1, 3, 2 and 4 rows (decode and verify) in turn:
    the counters' per-call epochs stay consistent; each call matches the stream-ordered kernels."""
    dtype = si.F16
    lens = [50, 90, 20, 70]
    cap = 128
    L = SeededLayer(6, 4, 1024, dtype)
    kb, vb = fill_cache(6, 4, lens, cap, dtype)
    plan = [("decode", [0]), ("decode", [1, 2, 3]), ("verify", [2]), ("decode", [3, 0]), ("verify", [1, 3]),
            ("decode", [0, 1, 2, 3]), ("decode", [2])]
    res = {}
    for mode in (ga.DISPATCH_MULTI, ga.DISPATCH_FUSED):
        kv = device_cache(kb, vb, lens, dtype)
        cfg = ga.config(dtype=dtype, dispatch=mode, kv_split=16)
        ws = ga.alloc_workspace(cfg, 4, cap)
        outs = []
        for step, (kind, slots) in enumerate(plan):
            if kind == "decode":
                outs.append(_run_decode(L, cfg, kv, _x(6, 4, step, (len(slots), 1024), dtype), dtype, slots=slots,
                                        ws=ws))
            else:
                outs.append(_run_verify(L, cfg, kv, _x(6, 4, step, (len(slots), 2, 1024), dtype), dtype, slots=slots,
                                        ws=ws))
        res[mode] = (outs, to_bits(kv.k), kv.lens.cpu().numpy(), kv.status.item())
    a, b = res[ga.DISPATCH_MULTI], res[ga.DISPATCH_FUSED]
    for oa, ob in zip(a[0], b[0]):
        assert np.max(np.abs(oa - ob)) <= AGREE * np.sqrt(np.mean(oa ** 2))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and a[3] == b[3] == 0


def test_one_workspace_for_calls_of_different_row_counts():
    """One workspace serves calls of 4, 64, 6 and 2 rows in turn (few-row kernels, then the
    equal-share attention whose merge counters sit where a smaller call's row table and
    projection were): every call equals the same call on a fresh zeroed workspace, bit for bit."""
    dtype = si.BF16
    lens = [int(v) for v in si.kv_lengths(9, 64, 200, 1500)]
    cap = 1536
    L = SeededLayer(9, 7, 1024, dtype)
    kb, vb = fill_cache(9, 7, lens, cap, dtype)
    plan = [[3, 9, 27, 40], list(range(64)), [1, 2, 3, 4, 5, 6], [60, 0]]
    cfg = ga.config(dtype=dtype)
    res = {}
    for shared in (True, False):
        kv = device_cache(kb, vb, lens, dtype)
        ws_shared = ga.alloc_workspace(cfg, 64, cap)
        outs = []
        for step, sl in enumerate(plan):
            ws = ws_shared if shared else ga.alloc_workspace(cfg, 64, cap)
            outs.append(_run_decode(L, cfg, kv, _x(9, 7, step, (len(sl), 1024), dtype), dtype, slots=sl, ws=ws))
        res[shared] = (outs, to_bits(kv.k), kv.lens.cpu().numpy(), kv.status.item())
    a, b = res[True], res[False]
    for oa, ob in zip(a[0], b[0]):
        assert np.all(np.isfinite(oa)) and np.array_equal(oa, ob)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and a[3] == b[3] == 0


@pytest.mark.parametrize("nq,nkv,k", [(16, 8, 8), (16, 8, 16), (16, 4, 4), (16, 4, 8), (16, 2, 4), (16, 2, 2)])
@pytest.mark.parametrize("split", [0, 128])
def test_verify_matrix_core_attention_groups_and_chunk_edges(nq, nkv, k, split):
    """Verify blocks on the matrix-core attention (one K/V stream per sequence and kv head) for
    2, 4 and 8 q heads per kv head: an empty cache, lengths whose appended rows straddle a
    128-key chunk boundary, one chunk ending exactly at the committed length, long ragged tails."""
    dtype = si.BF16 if k % 4 == 0 else si.F16
    lens = [0, 120, 128, 3, 517, 255][: max(2, 16 // k + 1)]
    cap = 640
    L = SeededLayer(11, nq * 100 + nkv * 10 + k, 1024, dtype, nq=nq, nkv=nkv)
    kb, vb = fill_cache(11, nkv * 10 + k, lens, cap, dtype, nkv=nkv)
    B = len(lens)
    slots = list(range(B))[::-1]
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = _x(11, nkv * 10 + k, 0, (B, k, 1024), dtype)
    cfg = ga.config(dtype=dtype, n_q_heads=nq, n_kv_heads=nkv, kv_split=split)
    got = _run_verify(L, cfg, kv, xb, dtype, slots=slots)
    want = oracle.verify(L.ocfg, L.ref, ref, xb, slots=slots)
    err = rel_err(got, want)
    print(f"verify mfma attention nq={nq} nkv={nkv} k={k} split={split} B={B}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + k for l in lens] and kv.status.item() == 0
    kg, vg = to_bits(kv.k), to_bits(kv.v)
    for s in range(B):
        check_rounded_rows(kg[s, :, lens[s]:lens[s] + k], ref.k[s, :, lens[s]:lens[s] + k], dtype)
        check_rounded_rows(vg[s, :, lens[s]:lens[s] + k], ref.v[s, :, lens[s]:lens[s] + k], dtype)
        assert np.array_equal(kg[s, :, :lens[s]], kb[s, :, :lens[s]])
        assert np.array_equal(kg[s, :, lens[s] + k:], kb[s, :, lens[s] + k:])


@pytest.mark.parametrize("B,k", [(1, 1), (3, 1), (6, 1), (2, 2), (2, 8)])
def test_multi_section_rotary_vs_oracle(B, k):
    """Three position components per sequence, rotary sections (16, 24, 24): decode (vector and
    matrix-core projections) and verify blocks; without positions the sections reduce to the
    one-position rotary, bit for bit."""
    dtype = si.BF16
    sections = (16, 24, 24)
    lens = [30, 250, 3, 77, 129, 0][:B]
    cap = 300
    L = SeededLayer(12, 10 * B + k, 1024, dtype)
    ocfg = oracle.BlockConfig(hidden=1024, dtype=dtype, mrope_sections=sections)
    kb, vb = fill_cache(12, B, lens, cap, dtype)
    pos3 = np.array([[100, 7, 2000, 5, 64, 0][:B], [3, 900, 11, 70, 1, 4][:B], [4000, 50, 9, 8, 300, 2][:B]], np.int32)
    cfg = ga.config(dtype=dtype, mrope_sections=sections)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    if k == 1:
        xb = _x(12, B, 0, (B, 1024), dtype)
        got = _run_decode(L, cfg, kv, xb, dtype, positions=pos3.ravel().tolist())
        want = oracle.decode(ocfg, L.ref, ref, xb, positions=pos3)
    else:
        xb = _x(12, B, 0, (B, k, 1024), dtype)
        got = _run_verify(L, cfg, kv, xb, dtype, positions=pos3.ravel().tolist())
        want = oracle.verify(ocfg, L.ref, ref, xb, positions=pos3)
    err = rel_err(got, want)
    print(f"mrope B={B} k={k}: {err:.3e}")
    assert err < TOL[dtype]
    kg = to_bits(kv.k)
    for s in range(B):
        check_rounded_rows(kg[s, :, lens[s]:lens[s] + k], ref.k[s, :, lens[s]:lens[s] + k], dtype)
    if k == 1:   # no positions: every component is the length, the one-position rotary
        a = _run_decode(L, cfg, device_cache(kb, vb, lens, dtype), xb, dtype)
        b = _run_decode(L, ga.config(dtype=dtype), device_cache(kb, vb, lens, dtype), xb, dtype)
        assert np.array_equal(a, b)
