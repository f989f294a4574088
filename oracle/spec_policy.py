"""Block-length and draft-recycling policy of the verify loop.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never calls it.

"Can CTC make Qwen3-ASR faster?" section 07 (strict whole-transcript
verification fails at the first mismatch even where the strings realign, so
verify in blocks, adapt the block length and recycle the aligned suffix) and
section 08 "Verifier, version 0" (at a mismatch append the target's correction,
crop, and recycle the part of the draft that realigns after it; choose the next
k from the draft's confidence: longer over low-entropy spans, shorter around
uncertain frames).  Section 11 Phase D step 5 adds both only once fixed-k
verification is token-identical: neither may change the committed transcript,
only how many target passes it takes.

Readings taken here (the pages give no formula):

* The draft is one token sequence D (the CTC transcript) with an uncertainty
  u[i] >= 0 per token (for example the entropy of its frames).  A round takes
  the next k tokens of D from a read position.
* Block length: with j the first remaining token whose uncertainty exceeds the
  threshold (j = the number of remaining tokens if none does), the block ends at
  that token: k = j + 1, clamped to [k_min, k_max] and to the tokens left (at
  least 1: with no draft left a round is a plain greedy step).
* Recycling: after a < k accepted tokens the target's correction c replaces
  D[pos + a].  If c equals one of the next `window` draft tokens D[pos + a + 1 ..
  pos + a + window], the draft tokens before the first such match were spurious
  and the draft realigns after the match: reading resumes just past it.  If the
  round failed at its first token (a = 0) and c equals one of the `window` draft
  tokens before pos (the nearest first), the previous round's realignment
  skipped a token the draft had dropped before it: reading resumes just past
  that match.  Otherwise D[pos + a] was a wrong token in the right place (a
  substitution) and reading resumes at pos + a + 1.  window = 0 is the
  substitution reading alone.
"""
from __future__ import annotations

from .spec_loop import TinyModel, speculative_round


def next_block_len(uncertainty, threshold: float, k_min: int, k_max: int) -> int:
    """The next block length from the uncertainties of the remaining draft tokens."""
    n = len(uncertainty)
    j = n
    for i, u in enumerate(uncertainty):
        if u > threshold:
            j = i
            break
    k = min(max(j + 1, k_min), k_max)
    return max(1, min(k, n))


def recycle_draft(draft, pos: int, k: int, accepted: int, correction, window: int) -> int:
    """Read position of the next round's draft after a round that took draft[pos:pos + k]."""
    if correction is None or accepted >= k:
        return pos + k
    miss = pos + accepted
    for j in range(miss + 1, min(miss + window, len(draft) - 1) + 1):      # spurious draft tokens
        if int(draft[j]) == int(correction):
            return j + 1
    if accepted == 0:                                                     # a token the draft dropped
        for j in range(min(pos, len(draft)) - 1, max(pos - window, 0) - 1, -1):
            if int(draft[j]) == int(correction):
                return j + 1
    return miss + 1


def speculative_decode(model: TinyModel, caches, last_token: int, draft, uncertainty, n_tokens: int,
                       threshold: float, k_min: int, k_max: int, window: int, pad: int = -1):
    """Rounds of verification until n_tokens are committed: block length from next_block_len,
    draft read position from recycle_draft.  Returns (committed tokens, the block lengths, the
    accepted counts).  Positions past the draft are padded with `pad` (an id that never wins)."""
    got, ks, accs = [], [], []
    pos, last = 0, last_token
    while len(got) < n_tokens:
        rest = list(draft[pos:])
        k = next_block_len(list(uncertainty[pos:]), threshold, k_min, k_max)
        block = (rest + [pad] * k)[:k]
        committed, a = speculative_round(model, caches, last, block)
        corr = committed[-1] if a < k else None
        pos = recycle_draft(draft, pos, k, a, corr, window)
        got += committed
        ks.append(k)
        accs.append(a)
        last = got[-1]
    return got, ks, accs
