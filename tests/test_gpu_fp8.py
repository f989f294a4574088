"""GPU parity of the FP8 (E4M3) KV cache against the fp64 oracle, through the C ABI: batched
decode and verify rows on the equal-share attention, every finite code, appended codes, the
byte-exact append, and the calls an FP8 cache does not take."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import (TOL, SeededLayer, check_codes, device_cache_e4m3, fill_cache_e4m3, oracle_cache_e4m3,
                        rel_err, to_dev)

pytestmark = pytest.mark.gpu


def _decode(L, cfg, kv, xb, dtype, slots=None, residual=None):
    B, H = xb.shape
    out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = ga.alloc_workspace(cfg, B, kv.c.capacity)
    ga.layer_decode(cfg, L.dev, kv, to_dev(xb, dtype), out, ws,
                    slots=None if slots is None else torch.tensor(slots, dtype=torch.int32, device="cuda"),
                    residual=None if residual is None else to_dev(residual, dtype))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", [si.BF16, si.F16])
@pytest.mark.parametrize("nkv", [8, 4])
@pytest.mark.parametrize("split", [0, 64])
def test_fp8_batched_decode_vs_oracle(dtype, nkv, split):
    lens = [0, 1, 17, 300, 129, 64, 511, 7, 250, 33]
    cap = 520
    slots = [3, 0, 5, 4, 1, 2, 9, 8, 6, 7]
    L = SeededLayer(21, nkv, 1024, dtype, nkv=nkv)
    kc, vc, ks, vs = fill_cache_e4m3(21, nkv, lens, cap, nkv=nkv)
    kv = device_cache_e4m3(kc, vc, lens, ks, vs)
    ref = oracle_cache_e4m3(kc, vc, lens, ks, vs)
    xb = si.activations(21, nkv, 0, len(lens), 1024, dtype)
    res = si.residual(21, nkv, 0, len(lens), 1024, dtype)
    got = _decode(L, ga.config(dtype=dtype, n_kv_heads=nkv, kv_split=split), kv, xb, dtype, slots=slots, residual=res)
    want = oracle.decode(L.ocfg, L.ref, ref, xb, slots=slots, residual_bits=res)
    err = rel_err(got, want)
    print(f"fp8 cache decode {dtype} nkv={nkv} split={split}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + 1 for l in lens] and kv.status.item() == 0
    kg, vg = kv.k.cpu().numpy(), kv.v.cpu().numpy()
    fk = check_codes(np.stack([kg[s, :, lens[s]] for s in range(len(lens))]),
                     np.stack([ref.k[s, :, lens[s]] for s in range(len(lens))]))
    fv = check_codes(np.stack([vg[s, :, lens[s]] for s in range(len(lens))]),
                     np.stack([ref.v[s, :, lens[s]] for s in range(len(lens))]))
    print(f"  appended codes differing: k {fk:.3%} v {fv:.3%}")
    for s in range(len(lens)):   # nothing else written
        assert np.array_equal(kg[s, :, :lens[s]], kc[s, :, :lens[s]])
        assert np.array_equal(kg[s, :, lens[s] + 1:], kc[s, :, lens[s] + 1:])


def test_fp8_every_finite_code_is_read_as_its_value():
    """Committed rows cycling through all 254 finite codes (both signs, subnormals, 448): the
    decode through the hardware conversion must read each as the oracle's value."""
    dtype = si.BF16
    lens = [254, 127, 300, 5, 64, 200]
    cap = 320
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    kc = np.zeros((6, 8, cap, 128), np.uint8)
    vc = np.zeros_like(kc)
    g = np.random.default_rng(3)
    for s in range(6):
        n = lens[s] * 8 * 128
        kc[s, :, :lens[s]] = np.resize(np.roll(finite, s), n).reshape(8, lens[s], 128)
        vc[s, :, :lens[s]] = g.choice(finite, size=(8, lens[s], 128))
    ks = np.full(8, 2.0 ** -9, np.float32)     # scores stay O(1) with codes up to 448
    vs = np.full(8, 2.0 ** -6, np.float32)
    L = SeededLayer(22, 0, 1024, dtype)
    kv = device_cache_e4m3(kc, vc, lens, ks, vs)
    ref = oracle_cache_e4m3(kc, vc, lens, ks, vs)
    xb = si.activations(22, 0, 0, 6, 1024, dtype)
    got = _decode(L, ga.config(dtype=dtype), kv, xb, dtype)
    want = oracle.decode(L.ocfg, L.ref, ref, xb)
    err = rel_err(got, want)
    print(f"fp8 every code: {err:.3e}")
    assert err < TOL[dtype]


@pytest.mark.parametrize("k", [2, 4])
def test_fp8_verify_rows_vs_oracle(k):
    dtype = si.BF16
    lens = [40, 0, 333, 129]
    cap = 400
    L = SeededLayer(23, k, 1024, dtype)
    kc, vc, ks, vs = fill_cache_e4m3(23, k, lens, cap)
    kv = device_cache_e4m3(kc, vc, lens, ks, vs)
    ref = oracle_cache_e4m3(kc, vc, lens, ks, vs)
    xb = si.activations(23, k, 0, 4 * k, 1024, dtype).reshape(4, k, 1024)
    out = torch.empty((4, k, 1024), dtype=torch.float32, device="cuda")
    cfg = ga.config(dtype=dtype)
    ga.layer_verify(cfg, L.dev, kv, to_dev(xb, dtype), out, ga.alloc_workspace(cfg, 4 * k, cap))
    torch.cuda.synchronize()
    want = oracle.verify(L.ocfg, L.ref, ref, xb)
    err = rel_err(out.cpu().numpy().astype(np.float64), want)
    print(f"fp8 verify k={k}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + k for l in lens]
    kg = kv.k.cpu().numpy()
    check_codes(np.concatenate([kg[s, :, lens[s]:lens[s] + k].ravel() for s in range(4)]),
                np.concatenate([ref.k[s, :, lens[s]:lens[s] + k].ravel() for s in range(4)]))


def test_fp8_append_is_byte_exact_and_unsupported_calls_refuse():
    cap, nkv = 32, 8
    g = np.random.default_rng(9)
    kc = g.integers(0, 256, (3, nkv, cap, 128)).astype(np.uint8)
    vc = g.integers(0, 256, (3, nkv, cap, 128)).astype(np.uint8)
    ks, vs = si.kv_scales(24, 0)
    lens0 = [3, 0, 29]
    kv = device_cache_e4m3(kc, vc, lens0, ks, vs)
    kn = g.integers(0, 256, (3, 4, nkv, 128)).astype(np.uint8)
    vn = g.integers(0, 256, (3, 4, nkv, 128)).astype(np.uint8)
    ga.kv_append(kv, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda())
    torch.cuda.synchronize()
    ref = oracle_cache_e4m3(kc, vc, lens0, ks, vs)
    oracle.kv_append(ref, kn, vn)
    assert np.array_equal(kv.k.cpu().numpy(), ref.k) and np.array_equal(kv.v.cpu().numpy(), ref.v)
    assert kv.lens.cpu().tolist() == ref.lens.tolist() == [7, 4, 29] and kv.status.item() == ga.STATUS_CAPACITY
    # few rows (vector-ALU path) and the fused dispatch do not take an FP8 cache
    dtype = si.BF16
    L = SeededLayer(24, 1, 1024, dtype)
    x = to_dev(si.activations(24, 1, 0, 2, 1024, dtype), dtype)
    out = torch.empty((2, 1024), dtype=torch.float32, device="cuda")
    cfg = ga.config(dtype=dtype)
    with pytest.raises(ga.AsrError) as e:
        ga.layer_decode(cfg, L.dev, kv, x, out, ga.alloc_workspace(cfg, 2, cap))
    assert e.value.code == -2
    assert kv.lens.cpu().tolist() == [7, 4, 29]
