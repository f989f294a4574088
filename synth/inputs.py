"""Seeded synthetic inputs for the decoder attention block.

This module is shared by the fp64 oracle, the GPU tests and the benchmark.  It
holds no arithmetic of the attention block itself: it only draws seeded normal
and integer values and stores each draw as the nearest 16-bit float, as raw
bit patterns (``numpy.uint16``), so that the oracle and the GPU path read the
very same bytes.

Workload shapes follow the pages: Qwen3-ASR-0.6B decoding a 60 s clip with
795 prompt tokens and 130 generated tokens ("Qwen3-ASR -- Latency & Bottleneck
Analysis", section 01 "Method & setup"), k-token speculative verification with
k in {4, 8, 16} ("Can CTC make Qwen3-ASR faster?", section 08 "Verifier,
version 0"), and batched serving of 30 s windows at 64 concurrent requests
("Baseten optimizes Qwen3-ASR 1.7B", sections "Our optimized Qwen3-ASR stack"
and "Throughput results").

Random streams: every tensor has its own NumPy PCG64 stream keyed by
``(1000 + stream, layer, tensor id, extra)``, the stream being a small
integer per workload or test family,, so any tensor can be
regenerated on its own.  Draws are fp64 ``standard_normal`` scaled to the
stated distribution, then rounded once, to nearest with ties to even, into the
workload's 16-bit type.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F16 = "f16"
BF16 = "bf16"

# tensor ids of the random streams
T_GAMMA_IN, T_WQKV, T_GAMMA_Q, T_GAMMA_K, T_WO = 0, 1, 2, 3, 4
T_KCACHE, T_VCACHE, T_X, T_LENS, T_ACCEPT, T_VCHOICE, T_RESID = 5, 6, 7, 8, 9, 10, 11
T_KVSCALE = 12
T_GAMMA_POST, T_WGATE, T_WUP, T_WDOWN, T_HIDDEN = 13, 14, 15, 16, 17

N_Q_HEADS = 16
N_KV_HEADS = 8
HEAD_DIM = 128
RMS_EPS = 1e-6
ROPE_THETA = 1e6

# The five workloads, by name.  Lengths are committed KV lengths before the
# step; "stream" keys the workload's random streams.
WORKLOADS = {
    "decode_bs1_1layer_kv64": dict(
        stream=1, name="single layer decode, bs1, fp16, KV 64", layers=1, batch=1,
        dtype=F16, hidden=1024, kv_len=(64, 64), steps=1),
    "decode_bs1_28layers_kv795": dict(
        stream=2, name="28-layer decode, bs1, fp16, KV 795->925 over 130 steps",
        layers=28, batch=1, dtype=F16, hidden=1024, kv_len=(795, 795), steps=130),
    "verify_bs1_28layers_kv795": dict(
        stream=3, name="28-layer verify k in {4,8,16}, bs1, fp16, committed 795",
        layers=28, batch=1, dtype=F16, hidden=1024, kv_len=(795, 795), verify_k=(4, 8, 16)),
    "ragged_batch64_h1024": dict(
        stream=4, name="28-layer ragged batched decode, 64 seqs, bf16, hidden 1024, KV U{200..1500}",
        layers=28, batch=64, dtype=BF16, hidden=1024, kv_len=(200, 1500), steps=1),
    "ragged_batch64_h2048": dict(
        stream=5, name="28-layer ragged batched decode, 64 seqs, bf16, hidden 2048, KV U{1024..4096}"
                       " + verify k=8 on 8 seqs",
        layers=28, batch=64, dtype=BF16, hidden=2048, kv_len=(1024, 4096),
        steps=1, verify_k=(8,), verify_seqs=8),
}


def seed_of(stream: int) -> int:
    return 1000 + int(stream)


def rng_for(stream: int, layer: int, tensor_id: int, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed_of(stream), int(layer), int(tensor_id), int(extra)])


def _f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of fp64 values, as uint16 bit patterns.

    bf16 keeps 8 significant bits with fp32's exponent range.  ``frexp`` gives
    a in [0.5, 1) * 2**e; scaling the fraction by 2**8 and ``rint`` (round half
    to even) keeps 8 bits exactly.  Below 2**-126 the spacing is fixed at
    2**-133.  Values of this generator never come near the overflow range.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    v = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    tiny = np.abs(a) < 2.0 ** -126
    if tiny.any():
        v[tiny] = np.ldexp(np.rint(np.ldexp(a[tiny], 133)), -133)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def to_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 draws once to the 16-bit type; return uint16 bit patterns."""
    if dtype == F16:
        # numpy converts float64 to float16 directly, rounding to nearest even
        return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return _f64_to_bf16_bits(a)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """Nearest FP8 E4M3 code (ties to even, saturating at +-448) of fp64 draws, as uint8.

    E4M3 keeps 4 significant bits; ``frexp`` gives a in [0.5, 1) * 2**e, so the
    fraction times 2**4, rounded half to even, keeps them.  Below 2**-6 the
    spacing is fixed at 2**-9.  The code is then assembled from the exponent
    and the 3 stored mantissa bits.
    """
    a = np.asarray(a, dtype=np.float64)
    sign = np.signbit(a)
    mag = np.minimum(np.abs(a), 448.0)
    m, e = np.frexp(mag)
    q = np.ldexp(np.rint(np.ldexp(m, 4)), e - 4)               # 4 significant bits
    sub = mag < 2.0 ** -6
    q = np.where(sub, np.ldexp(np.rint(np.ldexp(mag, 9)), -9), q)
    q = np.minimum(q, 448.0)
    m2, e2 = np.frexp(q)                                        # q = m2 * 2**e2, m2 in [0.5, 1)
    exp_field = np.where(q >= 2.0 ** -6, e2 - 1 + 7, 0)
    mant = np.where(exp_field > 0, np.rint((m2 * 2 - 1) * 8), np.rint(q * 2.0 ** 9))
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(q == 0, 0, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def normal_bits(stream, layer, tensor_id, extra, shape, std=1.0, mean=0.0, dtype=F16):
    g = rng_for(stream, layer, tensor_id, extra)
    return to_bits(mean + std * g.standard_normal(shape), dtype)


def layer_weights(stream: int, layer: int, hidden: int, dtype: str,
                  nq: int = N_Q_HEADS, nkv: int = N_KV_HEADS, d: int = HEAD_DIM,
                  gain_std: float = 0.02, gain_mean: float = 1.0, w_std: float = 0.02) -> dict:
    """Weights of one layer as bit patterns.

    Projections N(0, 0.02); norm gains 1 + N(0, 0.02).  ``w_qkv`` is
    [(nq + 2 nkv) d][hidden], rows q heads then k heads then v heads;
    ``w_o`` is [hidden][nq d]; both row-major [out][in].
    """
    nqkv = (nq + 2 * nkv) * d
    return dict(
        input_norm_w=normal_bits(stream, layer, T_GAMMA_IN, 0, (hidden,), gain_std, gain_mean, dtype),
        w_qkv=normal_bits(stream, layer, T_WQKV, 0, (nqkv, hidden), w_std, 0.0, dtype),
        q_norm_w=normal_bits(stream, layer, T_GAMMA_Q, 0, (d,), gain_std, gain_mean, dtype),
        k_norm_w=normal_bits(stream, layer, T_GAMMA_K, 0, (d,), gain_std, gain_mean, dtype),
        w_o=normal_bits(stream, layer, T_WO, 0, (hidden, nq * d), w_std, 0.0, dtype),
    )


def mlp_weights(stream: int, layer: int, hidden: int, intermediate: int, dtype: str,
                gain_std: float = 0.02, gain_mean: float = 1.0, w_std: float = 0.02) -> dict:
    """MLP weights of one layer as bit patterns: gate and up [intermediate][hidden], down
    [hidden][intermediate], N(0, 0.02); the post-attention norm gain 1 + N(0, 0.02)."""
    return dict(
        post_norm_w=normal_bits(stream, layer, T_GAMMA_POST, 0, (hidden,), gain_std, gain_mean, dtype),
        w_gate=normal_bits(stream, layer, T_WGATE, 0, (intermediate, hidden), w_std, 0.0, dtype),
        w_up=normal_bits(stream, layer, T_WUP, 0, (intermediate, hidden), w_std, 0.0, dtype),
        w_down=normal_bits(stream, layer, T_WDOWN, 0, (hidden, intermediate), w_std, 0.0, dtype),
    )


def hidden_f32(stream: int, layer: int, step: int, rows: int, hidden: int) -> np.ndarray:
    """fp32 hidden states entering the MLP (the attention block's fp32 output): N(0, 1) draws
    rounded to the nearest fp32."""
    return rng_for(stream, layer, T_HIDDEN, step).standard_normal((rows, hidden)).astype(np.float32)


def kv_rows(stream: int, layer: int, seq: int, length: int, dtype: str,
            nkv: int = N_KV_HEADS, d: int = HEAD_DIM):
    """Committed cache rows of one sequence: K, V bits, each [nkv][length][d], N(0, 1)."""
    k = normal_bits(stream, layer, T_KCACHE, seq, (nkv, length, d), 1.0, 0.0, dtype)
    v = normal_bits(stream, layer, T_VCACHE, seq, (nkv, length, d), 1.0, 0.0, dtype)
    return k, v


def kv_rows_e4m3(stream: int, layer: int, seq: int, length: int, k_scale, v_scale,
                 nkv: int = N_KV_HEADS, d: int = HEAD_DIM):
    """Committed FP8 cache rows of one sequence: codes of N(0, 1) draws divided by the
    per-kv-head scales, each [nkv][length][d] uint8 (the same draws as ``kv_rows``)."""
    ks = np.asarray(k_scale, np.float64).reshape(nkv, 1, 1)
    vs = np.asarray(v_scale, np.float64).reshape(nkv, 1, 1)
    k = rng_for(stream, layer, T_KCACHE, seq).standard_normal((nkv, length, d))
    v = rng_for(stream, layer, T_VCACHE, seq).standard_normal((nkv, length, d))
    return to_e4m3_codes(k / ks), to_e4m3_codes(v / vs)


def kv_scales(stream: int, layer: int, nkv: int = N_KV_HEADS):
    """Per-kv-head FP8 scales of K and V, fp32 values near 1/16 (so N(0, 1) rows use
    about the upper two thirds of the E4M3 range): 2^-4 * (1 + 0.25 u), u uniform in [0, 1)."""
    g = rng_for(stream, layer, T_KVSCALE, 0)
    return ((2.0 ** -4) * (1 + 0.25 * g.random(nkv))).astype(np.float32), \
           ((2.0 ** -4) * (1 + 0.25 * g.random(nkv))).astype(np.float32)


def kv_rows_many(stream, layer, seqs, lengths, dtype, nkv=N_KV_HEADS, d=HEAD_DIM, threads=None):
    """kv_rows for several sequences on a thread pool (NumPy releases the GIL)."""
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda sl: kv_rows(stream, layer, sl[0], sl[1], dtype, nkv, d),
                           zip(seqs, lengths)))


def kv_rows_e4m3_many(stream, layer, seqs, lengths, k_scale, v_scale, nkv=N_KV_HEADS, d=HEAD_DIM, threads=None):
    """kv_rows_e4m3 for several sequences on a thread pool."""
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda sl: kv_rows_e4m3(stream, layer, sl[0], sl[1], k_scale, v_scale, nkv, d),
                           zip(seqs, lengths)))


def activations(stream: int, layer: int, step: int, rows: int, hidden: int, dtype: str):
    """Hidden states entering the block at (layer, step): [rows][hidden], N(0, 1)."""
    return normal_bits(stream, layer, T_X, step, (rows, hidden), 1.0, 0.0, dtype)


def residual(stream: int, layer: int, step: int, rows: int, hidden: int, dtype: str):
    return normal_bits(stream, layer, T_RESID, step, (rows, hidden), 1.0, 0.0, dtype)


def kv_lengths(stream: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Committed lengths, uniform integers in [lo, hi] inclusive."""
    return rng_for(stream, 0, T_LENS, 0).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def accepted_prefix(stream: int, k: int, draw: int = 0) -> int:
    """Accepted draft prefix length, uniform in [0, k] inclusive."""
    return int(rng_for(stream, 0, T_ACCEPT, k * 1000 + draw).integers(0, k, endpoint=True))


def verify_choice(stream: int, batch: int, n: int) -> np.ndarray:
    """n distinct sequences of the batch, drawn without replacement."""
    return np.sort(rng_for(stream, 0, T_VCHOICE, 0).choice(batch, size=n, replace=False)).astype(np.int32)


T_EMBED, T_GAMMA_FINAL, T_WLM = 18, 19, 20


def head_weights(stream: int, hidden: int, vocab: int, dtype: str) -> dict:
    """Model-head weights as bit patterns: token embedding [vocab][hidden] N(0, 1), final norm
    gain 1 + N(0, 0.02), lm_head [vocab][hidden] N(0, 0.02)."""
    return dict(embed=normal_bits(stream, 0, T_EMBED, 0, (vocab, hidden), 1.0, 0.0, dtype),
                final_norm_w=normal_bits(stream, 0, T_GAMMA_FINAL, 0, (hidden,), 0.02, 1.0, dtype),
                w_lm=normal_bits(stream, 0, T_WLM, 0, (vocab, hidden), 0.02, 0.0, dtype))


# ------------------------------------------------------------------ synthetic drafts

T_DRAFT = 21


def draft_with_edits(stream: int, seq: int, transcript, rate: float, vocab: int, u_low: float = 0.3,
                     u_high: float = 3.0):
    """A stand-in for a CTC draft of `transcript` (the target's greedy tokens): each position is
    kept, or with probability `rate` substituted, preceded by an inserted token, or dropped (one
    third each), seeded by (stream, seq).  The per-token uncertainty is exponential with mean
    u_low, and u_high plus that noise at the draft token where an edit lands (the draft model
    knows its uncertain frames).  Returns (draft ids, uncertainties) as lists."""
    g = rng_for(stream, 0, T_DRAFT, seq)
    draft, unc = [], []
    for t in transcript:
        t = int(t)
        r = g.random()
        noise = float(g.exponential(u_low))
        if r < rate / 3:                         # substitution
            draft.append((t + 1 + int(g.integers(0, vocab - 1))) % vocab)
            unc.append(u_high + noise)
        elif r < 2 * rate / 3:                   # an inserted token before t
            draft += [int(g.integers(0, vocab)), t]
            unc += [u_high + noise, float(g.exponential(u_low))]
        elif r < rate:                           # t dropped: the next token carries the flag
            if unc:
                unc[-1] = max(unc[-1], u_high + noise)
        else:
            draft.append(t)
            unc.append(noise)
    return draft, unc


T_PAGES = 22


def page_table(stream: int, batch_cap: int, pages_per_seq: int, num_pages: int) -> np.ndarray:
    """A paged cache's table [batch_cap][pages_per_seq] int32: distinct pages of a pool of
    num_pages (>= batch_cap * pages_per_seq), in a seeded random order, so that neighbouring
    positions of a sequence sit in unrelated pages, as in a pool whose pages were handed out
    and returned by many requests."""
    assert num_pages >= batch_cap * pages_per_seq
    perm = rng_for(stream, 0, T_PAGES, num_pages).permutation(num_pages)
    return perm[:batch_cap * pages_per_seq].reshape(batch_cap, pages_per_seq).astype(np.int32)
