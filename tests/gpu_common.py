"""Helpers of the GPU parity tests: seeded layers on the device and in the oracle.

Both sides read the same 16-bit bit patterns from ``synth.inputs``; the GPU
side goes through the C ABI only.
"""
from __future__ import annotations

import numpy as np
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

TOL = {si.F16: 2e-3, si.BF16: 8e-3}   # max |err| / RMS(oracle output) per call


def tdt(dtype: str) -> torch.dtype:
    return torch.float16 if dtype == si.F16 else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt(dtype)).to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.max(np.abs(got - want)) / np.sqrt(np.mean(want * want)))


def check_rounded_rows(got_bits: np.ndarray, want_bits: np.ndarray, dtype: str, rel: float = 1e-5) -> float:
    """Cache rows the GPU rounded from its fp32 k/v against the oracle's rounding of the exact values.

    The GPU's fp32 value carries an absolute error of about 1e-6 of the row's RMS,
    which can move it across a rounding boundary of the 16-bit format.  So each
    stored element must lie within one unit in the last place of the oracle's
    value, or within ``rel`` * RMS of it (near zero, where a unit is tiny).
    Returns the fraction of elements that differ at all.
    """
    got_bits = np.asarray(got_bits, np.uint16)
    want_bits = np.asarray(want_bits, np.uint16)
    g, w = oracle.widen(got_bits, dtype), oracle.widen(want_bits, dtype)
    mag = want_bits & np.uint16(0x7FFF)
    ulp = oracle.widen((mag + np.uint16(1)).astype(np.uint16), dtype) - oracle.widen(mag, dtype)
    diff = np.abs(g - w)
    rms = np.sqrt(np.mean(w * w)) if w.size else 0.0
    ok = (diff <= ulp) | (diff <= rel * rms)
    assert ok.all(), f"{int((~ok).sum())} cache elements off by more than 1 ulp and {rel} RMS"
    return float(np.mean(got_bits != want_bits)) if got_bits.size else 0.0


class SeededLayer:
    """One layer's weights (device + oracle) from the seeded generator."""

    def __init__(self, stream, layer, hidden, dtype, nq=16, nkv=8, gain_mean=1.0):
        self.dtype = dtype
        self.bits = si.layer_weights(stream, layer, hidden, dtype, nq=nq, nkv=nkv, gain_mean=gain_mean)
        self.dev = ga.Weights(*(to_dev(self.bits[n], dtype) for n in
                                ("input_norm_w", "w_qkv", "q_norm_w", "k_norm_w", "w_o")))
        self.ref = oracle.LayerWeights.from_bits(self.bits, dtype)
        self.ocfg = oracle.BlockConfig(hidden=hidden, n_q_heads=nq, n_kv_heads=nkv, dtype=dtype)


def fill_cache(stream, layer, lens, capacity, dtype, nkv=8, seqs=None):
    """Host cache bits [batch_cap][nkv][capacity][128] with seeded rows below each length."""
    B = len(lens)
    k = np.zeros((B, nkv, capacity, 128), np.uint16)
    v = np.zeros_like(k)
    seqs = range(B) if seqs is None else seqs
    rows = si.kv_rows_many(stream, layer, list(seqs), [int(lens[s]) for s in seqs], dtype, nkv=nkv)
    for s, (kb, vb) in zip(seqs, rows):
        k[s, :, : lens[s]] = kb
        v[s, :, : lens[s]] = vb
    return k, v


def device_cache(kbits, vbits, lens, dtype) -> ga.KVLayer:
    return ga.KVLayer(to_dev(kbits, dtype), to_dev(vbits, dtype),
                      torch.tensor(np.asarray(lens, np.int32), device="cuda"),
                      torch.zeros(1, dtype=torch.int32, device="cuda"))


def oracle_cache(kbits, vbits, lens, dtype, seqs=None) -> oracle.KVCache:
    """Oracle cache holding the given sequences (all by default), slot order kept."""
    seqs = list(range(len(lens))) if seqs is None else list(seqs)
    c = oracle.KVCache(kbits[seqs].copy(), vbits[seqs].copy(), np.asarray(lens, np.int64)[seqs].copy(), dtype)
    return c


def fill_cache_e4m3(stream, layer, lens, capacity, nkv=8, seqs=None):
    """Host FP8 cache codes [batch_cap][nkv][capacity][128] and the per-kv-head scales."""
    ks, vs = si.kv_scales(stream, layer, nkv)
    B = len(lens)
    k = np.zeros((B, nkv, capacity, 128), np.uint8)
    v = np.zeros_like(k)
    for s in (range(B) if seqs is None else seqs):
        kc, vc = si.kv_rows_e4m3(stream, layer, s, int(lens[s]), ks, vs, nkv=nkv)
        k[s, :, : lens[s]] = kc
        v[s, :, : lens[s]] = vc
    return k, v, ks, vs


def device_cache_e4m3(kcodes, vcodes, lens, ks, vs) -> ga.KVLayer:
    return ga.KVLayer(torch.from_numpy(kcodes).cuda(), torch.from_numpy(vcodes).cuda(),
                      torch.tensor(np.asarray(lens, np.int32), device="cuda"),
                      torch.zeros(1, dtype=torch.int32, device="cuda"),
                      torch.from_numpy(np.asarray(ks, np.float32)).cuda(), torch.from_numpy(np.asarray(vs, np.float32)).cuda())


def oracle_cache_e4m3(kcodes, vcodes, lens, ks, vs, seqs=None) -> oracle.KVCache:
    seqs = list(range(len(lens))) if seqs is None else list(seqs)
    return oracle.KVCache(kcodes[seqs].copy(), vcodes[seqs].copy(), np.asarray(lens, np.int64)[seqs].copy(),
                          oracle.E4M3, 0, np.asarray(ks, np.float64), np.asarray(vs, np.float64))


def check_codes(got, want, max_frac=0.01):
    """Appended FP8 codes against the oracle's: the GPU quantises its fp32 value, the oracle the
    exact one, so a code may sit one step away where the two straddle a rounding boundary
    (codes of one sign are ordered by value, so one step is a difference of one); such
    straddles must stay rare.  Returns the fraction that differ."""
    got = np.asarray(got, np.uint8).astype(np.int64)
    want = np.asarray(want, np.uint8).astype(np.int64)
    same_sign = (got & 0x80) == (want & 0x80)
    g7, w7 = got & 0x7F, want & 0x7F
    # one step apart: same sign and adjacent magnitudes, or across zero (a zero code and the
    # smallest subnormal of either sign)
    ok = (same_sign & (np.abs(g7 - w7) <= 1)) | (~same_sign & (g7 + w7 <= 1))
    assert ok.all(), f"{int((~ok).sum())} codes more than one step from the oracle's"
    frac = float(np.mean(got != want)) if got.size else 0.0
    assert frac <= max_frac, f"{frac:.3%} of the codes differ from the oracle's"
    return frac
