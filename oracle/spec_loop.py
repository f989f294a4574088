"""fp64 CPU oracle of the greedy verify loop above the decoder.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never calls it.

"Can CTC make Qwen3-ASR faster?" section 03 ("Greedy exactness") and section
11 Phase A describe one speculative round of strict greedy verification:
score the draft's candidate positions in one causal pass of the target, take
the target's argmax at every position, accept the longest prefix of the
draft equal to it, emit the target's token at the first mismatch, and crop the
speculative cache to the committed prefix.  Section 11 step 3: the
distribution that verifies draft[i] comes from the position before it.

Reading taken here: a round starts from the last committed token p (its K/V
not yet in the cache) and feeds the block [p, draft[0], ..., draft[k-2]], so
block row i (the token before draft[i]) verifies draft[i].  With a accepted
drafts, the round commits draft[:a] and then, at a mismatch (a < k), the
target's token of row a; the cache keeps the block rows 0 .. a (p and the
accepted drafts) or all k rows when every draft is accepted, and the last
committed token starts the next round.  The committed count (a + 1 at a
mismatch, k otherwise) is the page's accept_greedy committed_length.

Written out: the token embedding (a row lookup), the final RMSNorm and the
lm_head with its argmax (ties to the smallest token id), the acceptance rule,
and a small reference model (embedding, decoder layers, final norm, lm_head)
with ordinary greedy decoding and speculative rounds, whose transcripts must
agree (the exactness claim of section 03).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attn_block import BlockConfig, kv_crop, rms_norm, rne16
from .decoder_layer import MlpConfig, decoder_layer_decode, decoder_layer_verify


@dataclass(frozen=True)
class HeadConfig:
    hidden: int = 1024
    vocab: int = 151936
    rms_eps: float = 1e-6
    dtype: str = "f16"


def embed(table_bits: np.ndarray, ids) -> np.ndarray:
    """The embedding rows of the token ids, as 16-bit patterns [len(ids)][H]."""
    return np.asarray(table_bits)[np.asarray(ids, np.int64)]


def lm_head_logits(cfg: HeadConfig, final_norm_w: np.ndarray, w_lm: np.ndarray, h: np.ndarray) -> np.ndarray:
    """logits[r] = W_lm RMSNorm(h[r]) (fp64), W_lm [V][H]."""
    return rms_norm(np.asarray(h, np.float64), final_norm_w, cfg.rms_eps) @ w_lm.T


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Index of the largest logit of each row; the smallest index among equal maxima."""
    return np.argmax(logits, axis=-1).astype(np.int64)


def accept_greedy(draft, target):
    """Strict greedy acceptance: target[i] is the target's argmax that verifies draft[i].

    Returns (accepted, correction, committed): the length of the longest draft prefix equal
    to the target's argmax; the target's token at the first mismatch (None when the whole
    draft is accepted); the number of tokens the round commits (accepted + 1 at a mismatch,
    len(draft) otherwise)."""
    k = len(draft)
    a = 0
    while a < k and int(draft[a]) == int(target[a]):
        a += 1
    if a < k:
        return a, int(target[a]), a + 1
    return a, None, k


@dataclass
class TinyModel:
    """A reference decoder-only model: embedding, layers, final norm, lm_head (fp64 values of
    16-bit weights; one attention-oracle cache per layer).  A layer's fp32 output enters the
    next layer rounded to the 16-bit type (the block takes 16-bit hidden states)."""
    acfg: BlockConfig
    mcfg: MlpConfig
    hcfg: HeadConfig
    embed_bits: np.ndarray          # [V][H] 16-bit patterns
    layers: list                    # [(LayerWeights, MlpWeights)]
    final_norm_w: np.ndarray        # [H]
    w_lm: np.ndarray                # [V][H]

    def forward(self, caches, tokens) -> np.ndarray:
        """A causal block of tokens (one token: a decode step) through every layer; the logits
        of every row."""
        x = embed(self.embed_bits, tokens)
        h = None
        for (aw, mw), c in zip(self.layers, caches):
            if len(tokens) == 1:
                h = decoder_layer_decode(self.acfg, aw, self.mcfg, mw, c, x)
            else:
                h = decoder_layer_verify(self.acfg, aw, self.mcfg, mw, c, x[None])[0]
            x = rne16(h, self.acfg.dtype)
        return lm_head_logits(self.hcfg, self.final_norm_w, self.w_lm, h)


def greedy_decode(model: TinyModel, caches, last_token: int, n: int) -> list:
    """Ordinary greedy decoding of n tokens after last_token, one forward per token."""
    out, tok = [], last_token
    for _ in range(n):
        tok = int(argmax_first(model.forward(caches, [tok]))[-1])
        out.append(tok)
    return out


def speculative_round(model: TinyModel, caches, last_token: int, draft):
    """One round from the last committed token with a draft of k tokens; returns the tokens
    the round commits (the last of them starts the next round) and the accepted count."""
    k = len(draft)
    lens0 = int(caches[0].lens[0])
    block = [last_token] + list(draft[:k - 1])
    target = argmax_first(model.forward(caches, block))
    a, corr, committed = accept_greedy(draft, target)
    kv_crop(caches, [lens0 + committed])
    return list(draft[:a]) + ([] if corr is None else [corr]), a
