"""fp64 CPU oracle of the decoder attention block.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path (the HIP library and its Python binding) never
calls it, and it imports nothing from the product path.

It is the plain definition of what one decoder attention block of a
Qwen3-ASR-style text decoder computes, written out in fp64 NumPy with no
blocking, fusion or reordering:

* input RMSNorm, then one fused q/k/v projection, then per-head RMSNorm of q
  and k, then rotary position embedding in full precision, then the KV-cache
  update, then grouped-query attention over the cache with a full-precision
  softmax, then the output projection.  The operation list is the one
  "Qwen3-ASR -- Latency & Bottleneck Analysis" gives for decoder attention in
  section 07 ("Why attention is 48.6% of decode": q/k/v projections, GQA
  repeat_kv, QK^T, softmax in fp32, AV, o_proj), with the norms of "Norms are
  real money at this size" (same section) and the rotary of section 03's
  module table ("rotary (MRoPE, fp32)").
* k-token verification scores k candidate positions in one causal pass over
  the committed cache; position i sees the committed prefix and the
  candidates up to and including i ("Can CTC make Qwen3-ASR faster?",
  section 03, "Speculative decoding: what work actually disappears?").
* cropping returns the cache to a committed prefix (same page, section 03
  "Greedy exactness" and section 11 Phase D, transactional commit/crop).

Readings taken where the pages are silent (each one is listed with its reason
in the design notes): rotate-half rotary pairing (t, t + d/2); one scalar
position per token, so the multi-section rotary reduces to the 1-D form; the
new token sits at position ``lens`` and attends to itself; attention reads the
appended K/V as stored (rounded once to the cache's 16-bit type); scale
1/sqrt(d); q head i uses kv head i // (nq / nkv); RMSNorm is
x * g / sqrt(mean(x^2) + eps) with the same eps for all norms; no biases.

Inputs are 16-bit bit patterns (``uint16``) widened exactly to fp64; every
intermediate stays in fp64, and the only rounding is the one into the cache.

The cache may also hold FP8 codes (E4M3: 1 sign, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, one NaN pattern per sign) with one fp32 scale
per kv head for K and one for V: a cached value is scale * decode(code), and a
row enters the cache as the code nearest to value / scale, ties to the even
code, magnitudes past the largest finite value (448) saturating to it.  This
follows "Baseten optimizes Qwen3-ASR 1.7B", section "KV cache quantization"
(the cache in FP8, the attention arithmetic at full precision); the E4M3
layout and the saturating conversion are the readings taken where that page
is silent.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F16 = "f16"
BF16 = "bf16"
E4M3 = "e4m3"

STATUS_CAPACITY = 1   # an append would pass the cache capacity: rows skipped, output NaN
STATUS_CROP_GROW = 2  # a crop asked for a length above the current one: ignored


# ----------------------------------------------------------------------------
# 16-bit formats, from their bit patterns

def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of 16-bit bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


_TABLES: dict = {}


def _magnitude_table(dtype: str):
    """Non-negative finite patterns in ascending order, then the infinity pattern.

    For IEEE-style formats the non-negative patterns 0 .. max-finite are
    ordered by value.  Infinity is placed where the next pattern would be,
    with the value max + ulp(max), so that round-to-nearest-even overflows to
    infinity exactly when IEEE 754 says it does.
    """
    if dtype not in _TABLES:
        if dtype == F16:
            max_pat, inf_pat, inf_val = 0x7BFF, 0x7C00, 65536.0
        elif dtype == BF16:
            max_pat, inf_pat, inf_val = 0x7F7F, 0x7F80, 2.0 ** 128
        else:
            raise ValueError(dtype)
        pats = np.arange(0, max_pat + 1, dtype=np.uint32).astype(np.uint16)
        vals = np.append(widen(pats, dtype), inf_val)
        pats = np.append(pats, np.uint16(inf_pat))
        _TABLES[dtype] = (vals, pats)
    return _TABLES[dtype]


def rne16(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest 16-bit value, ties to the even pattern.

    Works from the table of representable magnitudes: find the two
    neighbours, keep the nearer, and on an exact tie keep the one whose
    pattern is even.  The sign bit is copied (so -0.0 stays -0.0).
    """
    a = np.asarray(a, dtype=np.float64)
    vals, pats = _magnitude_table(dtype)
    mag = np.abs(a)
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pats[hi] % 2 == 0))
    out = np.where(pick_hi, pats[hi], pats[lo]).astype(np.uint16)
    out = np.where(mag >= vals[-1], pats[-1], out)          # at or past infinity
    out = np.where(np.signbit(a), out | np.uint16(0x8000), out).astype(np.uint16)
    nan_pat = np.uint16(0x7E00 if dtype == F16 else 0x7FC0)
    return np.where(np.isnan(a), nan_pat, out).astype(np.uint16)


# ----------------------------------------------------------------------------
# FP8 E4M3 codes

E4M3_MAX = 448.0


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 value of E4M3 codes (uint8): sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0; exponent 0 is the subnormal range
    m * 2^-9; exponent 15 with mantissa 7 is NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def rne_e4m3(a: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of fp64 values, ties to the even code; magnitudes past
    448 saturate to 448 (there is no infinity to round to); NaN to the NaN code.

    Works from the ascending table of the 127 non-negative finite codes, as
    ``rne16`` does for the 16-bit formats.
    """
    a = np.asarray(a, dtype=np.float64)
    pats = np.arange(0, 0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: 0 .. 448 ascending
    vals = e4m3_value(pats)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pats[hi] % 2 == 0))
    out = np.where(pick_hi, pats[hi], pats[lo]).astype(np.uint8)
    out = np.where(np.signbit(a), out | np.uint8(0x80), out).astype(np.uint8)
    return np.where(np.isnan(a), np.uint8(0x7F), out).astype(np.uint8)


# ----------------------------------------------------------------------------
# configuration, weights, cache

@dataclass(frozen=True)
class BlockConfig:
    hidden: int = 1024
    n_q_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    dtype: str = F16
    # multi-section rotary: rotary pairs [0, s0) turn by position component 0, the next s1 by
    # component 1, the last s2 by component 2 (s0 + s1 + s2 = head_dim / 2); () = one position
    mrope_sections: tuple = ()


@dataclass
class LayerWeights:
    """One layer's weights widened to fp64 (inputs are 16-bit patterns)."""
    input_norm_w: np.ndarray   # [H]
    w_qkv: np.ndarray          # [(nq + 2 nkv) d][H], rows q | k | v, head-major
    q_norm_w: np.ndarray       # [d]
    k_norm_w: np.ndarray       # [d]
    w_o: np.ndarray            # [H][nq d]

    @classmethod
    def from_bits(cls, bits: dict, dtype: str) -> "LayerWeights":
        return cls(**{name: widen(bits[name], dtype) for name in
                      ("input_norm_w", "w_qkv", "q_norm_w", "k_norm_w", "w_o")})


@dataclass
class KVCache:
    """One layer's cache: K and V as codes [batch_cap][nkv][capacity][d].

    16-bit caches hold ``uint16`` bit patterns of ``dtype``; FP8 caches
    (``dtype`` E4M3) hold ``uint8`` codes and the per-kv-head scales
    ``k_scale``, ``v_scale`` (fp32 values)."""
    k: np.ndarray
    v: np.ndarray
    lens: np.ndarray           # [batch_cap] committed lengths
    dtype: str
    status: int = 0
    k_scale: np.ndarray = None   # [nkv], E4M3 caches only
    v_scale: np.ndarray = None

    @classmethod
    def empty(cls, batch_cap, n_kv_heads, capacity, head_dim, dtype, k_scale=None, v_scale=None):
        shape = (batch_cap, n_kv_heads, capacity, head_dim)
        ct = np.uint8 if dtype == E4M3 else np.uint16
        return cls(np.zeros(shape, ct), np.zeros(shape, ct), np.zeros(batch_cap, np.int64), dtype, 0,
                   None if k_scale is None else np.asarray(k_scale, np.float64),
                   None if v_scale is None else np.asarray(v_scale, np.float64))

    @property
    def capacity(self) -> int:
        return self.k.shape[2]

    def copy(self) -> "KVCache":
        return KVCache(self.k.copy(), self.v.copy(), self.lens.copy(), self.dtype, self.status,
                       self.k_scale, self.v_scale)

    def encode(self, which: str, rows: np.ndarray) -> np.ndarray:
        """Codes of rows [nkv][n][d] (or [nkv][d]) as this cache stores them."""
        if self.dtype != E4M3:
            return rne16(rows, self.dtype)
        sc = self.k_scale if which == "k" else self.v_scale
        sc = sc.reshape((-1,) + (1,) * (rows.ndim - 1))
        return rne_e4m3(rows / sc)

    def values(self, which: str, g: int, codes: np.ndarray) -> np.ndarray:
        """fp64 values of codes of kv head g."""
        if self.dtype != E4M3:
            return widen(codes, self.dtype)
        sc = self.k_scale[g] if which == "k" else self.v_scale[g]
        return sc * e4m3_value(codes)


# ----------------------------------------------------------------------------
# the steps of the block

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x * gain / sqrt(mean(x^2) + eps), over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * gain / np.sqrt(ms + eps)


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_t = theta^(-2t/d), t = 0 .. d/2 - 1 (a geometric ladder from 1)."""
    t = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * t / head_dim)


def rope(u: np.ndarray, pos, theta: float, sections=()) -> np.ndarray:
    """Rotate pairs (t, t + d/2) of the last axis by the angle pos * omega_t.

    ``pos`` broadcasts against ``u.shape[:-1]``.  With ``sections`` (s0, s1, s2), ``pos`` has
    a trailing axis of three position components and pair t turns by component c(t): 0 for
    t < s0, 1 for t < s0 + s1, 2 after ("MRoPE" of the Latency page's section 03 table).
    """
    d = u.shape[-1]
    half = d // 2
    om = rope_frequencies(d, theta)
    if sections:
        assert sum(sections) == half
        comp = np.repeat(np.arange(3), sections)                       # component of each pair
        p = np.asarray(pos, dtype=np.float64)
        ang = np.take(p, comp, axis=-1) * om                            # [..., half]
    else:
        ang = np.asarray(pos, dtype=np.float64)[..., None] * om
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _split_qkv(qkv: np.ndarray, cfg: BlockConfig):
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = qkv[..., : nq * d].reshape(qkv.shape[:-1] + (nq, d))
    k = qkv[..., nq * d: (nq + nkv) * d].reshape(qkv.shape[:-1] + (nkv, d))
    v = qkv[..., (nq + nkv) * d:].reshape(qkv.shape[:-1] + (nkv, d))
    return q, k, v


def _softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def decode(cfg: BlockConfig, w: LayerWeights, cache: KVCache, x_bits: np.ndarray,
           slots=None, positions=None, residual_bits=None) -> np.ndarray:
    """One-token decode for B rows (each row a distinct sequence slot).

    Row i works on slot ``slots[i]`` (default i) at position
    ``positions[i]`` (default the slot's length; with multi-section rotary ``positions`` is
    [3][B], the components of row i at ``positions[:, i]``): it computes q, k, v, appends
    k and v at index lens[slot], attends over lens[slot] + 1 positions and
    returns out[i] = W_o a (+ residual).  lens[slot] grows by one.  A row whose
    append would pass the capacity is skipped: NaN output, the capacity status
    bit set, its length unchanged.  Rows are handled one at a time here, as a
    sequence of single-row computations.
    """
    x = widen(x_bits, cfg.dtype)
    B = x.shape[0]
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = nq // nkv
    res = widen(residual_bits, cfg.dtype) if residual_bits is not None else None
    out = np.empty((B, cfg.hidden), np.float64)
    for i in range(B):
        s = int(slots[i]) if slots is not None else i
        L = int(cache.lens[s])
        h = rms_norm(x[i], w.input_norm_w, cfg.rms_eps)
        q, k, v = _split_qkv(w.w_qkv @ h, cfg)
        q = rms_norm(q, w.q_norm_w, cfg.rms_eps)
        k = rms_norm(k, w.k_norm_w, cfg.rms_eps)
        if cfg.mrope_sections:   # positions [3][B]: the row's three components
            p = np.asarray(positions, np.int64)[:, i] if positions is not None else np.full(3, L)
            q = rope(q, p[None, :], cfg.rope_theta, cfg.mrope_sections)
            k = rope(k, p[None, :], cfg.rope_theta, cfg.mrope_sections)
        else:
            p = int(positions[i]) if positions is not None else L
            q = rope(q, p, cfg.rope_theta)
            k = rope(k, p, cfg.rope_theta)
        if L + 1 > cache.capacity:
            cache.status |= STATUS_CAPACITY
            out[i] = np.nan
            continue
        cache.k[s, :, L, :] = cache.encode("k", k)
        cache.v[s, :, L, :] = cache.encode("v", v)
        n_vis = L + 1
        a = np.empty((nq, d))
        for head in range(nq):
            g = head // group
            K = cache.values("k", g, cache.k[s, g, :n_vis, :])
            V = cache.values("v", g, cache.v[s, g, :n_vis, :])
            wts = _softmax(K @ q[head] / math.sqrt(d))
            a[head] = wts @ V
        out[i] = w.w_o @ a.reshape(nq * d)
        if res is not None:
            out[i] += res[i]
        cache.lens[s] = n_vis
    return out


def verify(cfg: BlockConfig, w: LayerWeights, cache: KVCache, x_bits: np.ndarray,
           slots=None, positions=None, residual_bits=None) -> np.ndarray:
    """k-token causal verification block for B sequences: x is [B][k][H].

    For each sequence the k rows are processed as one block: one [k x H]
    projection, k appends at lens .. lens + k - 1, and a causally masked
    [k x (lens + k)] score matrix per query head, where row r sees positions
    0 .. lens + r.  Rotary positions are ``positions[b] + r`` (default
    lens + r).  lens grows by k.
    """
    x = widen(x_bits, cfg.dtype)
    B, kk, _ = x.shape
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = nq // nkv
    res = widen(residual_bits, cfg.dtype) if residual_bits is not None else None
    out = np.empty((B, kk, cfg.hidden), np.float64)
    for b in range(B):
        s = int(slots[b]) if slots is not None else b
        L = int(cache.lens[s])
        Hn = rms_norm(x[b], w.input_norm_w, cfg.rms_eps)                # [k][H]
        Q, K_new, V_new = _split_qkv(Hn @ w.w_qkv.T, cfg)               # [k][heads][d]
        Q = rms_norm(Q, w.q_norm_w, cfg.rms_eps)
        K_new = rms_norm(K_new, w.k_norm_w, cfg.rms_eps)
        if cfg.mrope_sections:   # every component of row r advances by r
            p0 = np.asarray(positions, np.int64)[:, b] if positions is not None else np.full(3, L)
            pos = p0[None, :] + np.arange(kk)[:, None]                  # [k][3]
            Q = rope(Q, pos[:, None, :], cfg.rope_theta, cfg.mrope_sections)
            K_new = rope(K_new, pos[:, None, :], cfg.rope_theta, cfg.mrope_sections)
        else:
            p0 = int(positions[b]) if positions is not None else L
            pos = p0 + np.arange(kk)
            Q = rope(Q, pos[:, None], cfg.rope_theta)
            K_new = rope(K_new, pos[:, None], cfg.rope_theta)
        if L + kk > cache.capacity:
            cache.status |= STATUS_CAPACITY
            out[b] = np.nan
            continue
        cache.k[s, :, L:L + kk, :] = cache.encode("k", K_new.transpose(1, 0, 2))
        cache.v[s, :, L:L + kk, :] = cache.encode("v", V_new.transpose(1, 0, 2))
        n_all = L + kk
        visible = np.arange(n_all)[None, :] <= (L + np.arange(kk))[:, None]   # [k][L + k]
        A = np.empty((kk, nq, d))
        for head in range(nq):
            g = head // group
            K = cache.values("k", g, cache.k[s, g, :n_all, :])
            V = cache.values("v", g, cache.v[s, g, :n_all, :])
            S = (Q[:, head, :] @ K.T) / math.sqrt(d)
            S = np.where(visible, S, -np.inf)
            A[:, head, :] = _softmax(S) @ V
        out[b] = A.reshape(kk, nq * d) @ w.w_o.T
        if res is not None:
            out[b] += res[b]
        cache.lens[s] = n_all
    return out


def mixed(cfg: BlockConfig, w: LayerWeights, cache: KVCache, x_bits: np.ndarray, n_per_seq,
          slots=None, positions=None, residual_bits=None) -> np.ndarray:
    """Decode rows and verify blocks of different sizes in one call: x is [sum(n_per_seq)][H].

    "Can CTC make Qwen3-ASR faster?", section 08 (Verifier, version 0) picks the
    block length of each sequence from the draft's confidence, so the sequences
    of one batch carry blocks of different k (k = 1: a decode step).  Sequence b
    owns the n_per_seq[b] consecutive rows after those of sequences 0 .. b - 1,
    and they are exactly its verify block (rows appended at lens .. lens + k - 1,
    row r seeing positions 0 .. lens + r, rotary at positions[b] + r).
    Positions: [B] (one per sequence), or [3][B] with multi-section rotary.
    """
    n_per_seq = [int(n) for n in n_per_seq]
    x_bits = np.asarray(x_bits)
    out = np.empty((sum(n_per_seq), cfg.hidden), np.float64)
    row = 0
    for b, n in enumerate(n_per_seq):
        s = int(slots[b]) if slots is not None else b
        if positions is None:
            pos = None
        elif cfg.mrope_sections:
            pos = np.asarray(positions, np.int64)[:, b:b + 1]
        else:
            pos = [int(positions[b])]
        res = residual_bits[None, row:row + n] if residual_bits is not None else None
        out[row:row + n] = verify(cfg, w, cache, x_bits[None, row:row + n], slots=[s], positions=pos,
                                  residual_bits=res)[0]
        row += n
    return out


def kv_append(cache: KVCache, k_bits: np.ndarray, v_bits: np.ndarray, slots=None) -> None:
    """Copy given rows (16-bit patterns or E4M3 codes) into the cache: k_bits, v_bits are [B][n][nkv][d].

    Rows of sequence b go to positions lens .. lens + n - 1 of slot
    ``slots[b]``; lens grows by n.  A sequence whose rows would pass the
    capacity is skipped and the capacity status bit set.
    """
    ct = np.uint8 if cache.dtype == E4M3 else np.uint16
    k_bits = np.asarray(k_bits, ct)
    v_bits = np.asarray(v_bits, ct)
    B, n = k_bits.shape[:2]
    for b in range(B):
        s = int(slots[b]) if slots is not None else b
        L = int(cache.lens[s])
        if L + n > cache.capacity:
            cache.status |= STATUS_CAPACITY
            continue
        cache.k[s, :, L:L + n, :] = k_bits[b].transpose(1, 0, 2)
        cache.v[s, :, L:L + n, :] = v_bits[b].transpose(1, 0, 2)
        cache.lens[s] = L + n


def kv_crop(caches, new_lens) -> None:
    """Set every layer's lens to new_lens; cached data is left as it is.

    Only shrinking (or keeping) is allowed: a slot whose new length is
    negative or above its current one keeps its length and the layer's
    crop-grow status bit is set.
    """
    new_lens = np.asarray(new_lens)
    for c in caches:
        for b in range(len(c.lens)):
            nl = int(new_lens[b])
            if 0 <= nl <= c.lens[b]:
                c.lens[b] = nl
            else:
                c.status |= STATUS_CROP_GROW
