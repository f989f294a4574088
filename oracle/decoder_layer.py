"""fp64 CPU oracle of the rest of the decoder layer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never calls it, and it imports nothing from the
product path (only the attention-block oracle next to it).

"Qwen3-ASR -- Latency & Bottleneck Analysis" splits each decoder layer into
attention, MLP and the norms (section 03 module table: decoder MLP 5.114 ms per
token, memory-bound at 529 MB/token; section 06 row 2; section 07 "Norms are
real money at this size": the input and post-attention RMSNorms of every
layer).  Written out here, per row, as plain definitions in fp64:

* the post-attention RMSNorm: y = h * g_post / sqrt(mean(h^2) + eps);
* the MLP: out = W_down (silu(W_gate y) * (W_up y)), silu(u) = u / (1 + e^-u);
* the residual: the layer's output is h + out, where h = x + attention(x) is
  the attention block's output with the layer input as its residual.

Readings where the pages are silent: the MLP is the gated SiLU form with three
equal-sized matrices (the 529 MB/token of section 03 is exactly three 1024 x
3072 16-bit matrices per layer over 28 layers, so the intermediate width is
3072 at hidden 1024; 6144 at hidden 2048, the same ratio); no biases; the
post-attention norm uses the same eps as the other norms.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attn_block import BlockConfig, KVCache, LayerWeights, decode, mixed, rms_norm, verify, widen


@dataclass(frozen=True)
class MlpConfig:
    hidden: int = 1024
    intermediate: int = 3072
    rms_eps: float = 1e-6
    dtype: str = "f16"


@dataclass
class MlpWeights:
    """One layer's MLP weights widened to fp64."""
    post_norm_w: np.ndarray   # [H]
    w_gate: np.ndarray        # [I][H]
    w_up: np.ndarray          # [I][H]
    w_down: np.ndarray        # [H][I]

    @classmethod
    def from_bits(cls, bits: dict, dtype: str) -> "MlpWeights":
        return cls(**{n: widen(bits[n], dtype) for n in ("post_norm_w", "w_gate", "w_up", "w_down")})


def silu(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(u), written as u / (1 + exp(-u))."""
    return u / (1.0 + np.exp(-u))


def mlp(cfg: MlpConfig, w: MlpWeights, h: np.ndarray) -> np.ndarray:
    """The layer's output h + MLP(RMSNorm(h)) for rows h [rows][H] (fp64 values)."""
    h = np.asarray(h, np.float64)
    y = rms_norm(h, w.post_norm_w, cfg.rms_eps)
    act = silu(y @ w.w_gate.T) * (y @ w.w_up.T)
    return h + act @ w.w_down.T


def decoder_layer_decode(acfg: BlockConfig, aw: LayerWeights, mcfg: MlpConfig, mw: MlpWeights, cache: KVCache,
                         x_bits: np.ndarray, slots=None, positions=None) -> np.ndarray:
    """One whole decoder layer for B one-token rows: h = x + attention(x), then h + MLP(h).
    Rows whose append would pass the capacity come out NaN (as from the attention block)."""
    h = decode(acfg, aw, cache, x_bits, slots=slots, positions=positions, residual_bits=x_bits)
    return mlp(mcfg, mw, h)


def decoder_layer_verify(acfg: BlockConfig, aw: LayerWeights, mcfg: MlpConfig, mw: MlpWeights, cache: KVCache,
                         x_bits: np.ndarray, slots=None, positions=None) -> np.ndarray:
    """The k-token verify block through a whole decoder layer: x is [B][k][H]."""
    h = verify(acfg, aw, cache, x_bits, slots=slots, positions=positions, residual_bits=x_bits)
    B, k, H = h.shape
    return mlp(mcfg, mw, h.reshape(B * k, H)).reshape(B, k, H)


def decoder_layer_mixed(acfg: BlockConfig, aw: LayerWeights, mcfg: MlpConfig, mw: MlpWeights, cache: KVCache,
                        x_bits: np.ndarray, n_per_seq, slots=None, positions=None) -> np.ndarray:
    """Decode rows and verify blocks of per-sequence sizes through a whole decoder layer:
    x is [sum(n_per_seq)][H] (the attention block of ``mixed``, then the MLP row by row)."""
    h = mixed(acfg, aw, cache, x_bits, n_per_seq, slots=slots, positions=positions, residual_bits=x_bits)
    return mlp(mcfg, mw, h)
