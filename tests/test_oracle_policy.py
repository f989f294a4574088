"""Pins of the oracle's block-length and draft-recycling policy ("Can CTC make Qwen3-ASR
faster?", section 07 and section 08 "Verifier, version 0": adaptive block length from the draft's
confidence, recycling of the draft suffix that realigns after a correction; section 11 Phase D
step 5: neither may change the transcript).  Hand-worked cases of both rules, the transcript of
whole speculative decodes with drafts carrying substitutions, insertions and deletions (always
the greedy one), and the rounds that recycling and adaptive blocks save on such drafts."""
import pytest

from oracle import greedy_decode, next_block_len, recycle_draft, speculative_decode

from test_oracle_loop import _model


def test_block_length_ends_at_the_first_uncertain_token():
    u = [0.1, 0.2, 0.1, 0.3, 0.2, 2.5, 0.1, 0.1]
    assert next_block_len(u, 1.0, 2, 16) == 6            # tokens 0..5, the uncertain one included
    assert next_block_len(u, 3.0, 2, 16) == 8            # none uncertain: every token left
    assert next_block_len(u + [0.0] * 30, 3.0, 2, 16) == 16   # ... up to k_max
    assert next_block_len([5.0] + u, 1.0, 1, 16) == 1    # the first token uncertain
    assert next_block_len([5.0] + u, 1.0, 4, 16) == 4    # ... at least k_min
    assert next_block_len([0.1, 0.1, 0.1], 1.0, 4, 16) == 3   # never past the draft
    assert next_block_len([], 1.0, 4, 16) == 1           # no draft left: a greedy step
    assert next_block_len([1.0, 1.0, 2.0], 1.0, 1, 8) == 3    # equal to the threshold is not above it


def test_recycle_cases():
    D = [10, 11, 12, 13, 14, 15]
    assert recycle_draft(D, 0, 4, 4, None, 2) == 4                 # all accepted
    assert recycle_draft(D, 0, 4, 1, 99, 2) == 2                   # substitution of D[1]
    ins = [10, 77, 11, 12, 13]                                     # 77 inserted before 11
    assert recycle_draft(ins, 0, 4, 1, 11, 1) == 3                 # realigned after 11
    assert recycle_draft(ins, 0, 4, 1, 11, 0) == 2                 # window 0: substitution reading
    two = [10, 77, 78, 11, 12]
    assert recycle_draft(two, 0, 4, 1, 11, 1) == 2                 # the match lies past the window
    assert recycle_draft(two, 0, 4, 1, 11, 2) == 4
    rep = [10, 5, 11, 11, 12]
    assert recycle_draft(rep, 0, 4, 1, 11, 3) == 3                 # the first match
    assert recycle_draft(D, 2, 3, 2, 99, 4) == 5                   # a round that started at pos 2
    assert recycle_draft(D, 4, 2, 1, 15, 4) == 6                   # miss at the last-but-one token
    assert recycle_draft(D, 5, 1, 0, 7, 4) == 6                    # miss at the last token
    # a dropped token: the draft skips t3 (D = t0 t1 t2 t4 t5 ...); the first round misses t3 and
    # takes the substitution reading (resume at 4); the next round fails at once with t4 = draft[3]
    drop = [20, 21, 22, 24, 25, 26, 27]
    assert recycle_draft(drop, 0, 4, 3, 23, 2) == 4
    assert recycle_draft(drop, 4, 4, 0, 24, 2) == 4                # realigned: resume at 25
    assert recycle_draft(drop, 4, 4, 0, 24, 0) == 5                # window 0: substitution reading
    assert recycle_draft(drop, 4, 4, 1, 24, 2) == 6                # only a round that failed at once
    assert recycle_draft([5, 9, 5, 1, 2, 3], 3, 2, 0, 5, 3) == 3   # the nearest earlier match
    assert recycle_draft([5, 9, 6, 1, 2, 3], 3, 2, 0, 5, 2) == 4   # ... within the window only


def _edit(seq, kind, at, vocab):
    """The greedy transcript with one edit at position `at`."""
    s = list(seq)
    if kind == "sub":
        s[at] = (s[at] + 1) % vocab
    elif kind == "ins":
        s.insert(at, (s[at] + 7) % vocab)
    elif kind == "del":
        del s[at]
    return s


@pytest.mark.parametrize("edits", [[], [("sub", 3)], [("ins", 2)], [("del", 4)],
                                   [("sub", 1), ("ins", 6), ("del", 11)]])
@pytest.mark.parametrize("window,k_min,k_max", [(0, 4, 4), (2, 2, 8), (4, 1, 16)])
def test_speculative_decode_with_recycling_commits_the_greedy_transcript(edits, window, k_min, k_max):
    model, caches = _model(21)
    ref = [c.copy() for c in caches]
    n = 16
    want = greedy_decode(model, ref, 3, n + 8)
    draft = want
    for kind, at in edits[::-1]:
        draft = _edit(draft, kind, at, model.hcfg.vocab)
    unc = [0.0] * len(draft)
    got, ks, accs = speculative_decode(model, caches, 3, draft, unc, n, 1.0, k_min, k_max, window)
    assert got[:n] == want[:n]
    assert all(k_min <= k <= k_max or k < k_min for k in ks) and all(a <= k for a, k in zip(accs, ks))
    assert int(caches[0].lens[0]) == 7 + len(got)


def test_recycling_realigns_after_an_insertion():
    """An inserted draft token: with a window the round after the correction accepts its whole
    block again; the substitution reading stays one token out of step and keeps missing."""
    model, caches0 = _model(22)
    want = greedy_decode(model, [c.copy() for c in caches0], 4, 30)
    draft = _edit(want, "ins", 3, model.hcfg.vocab)
    unc = [0.0] * len(draft)
    got1, ks1, acc1 = speculative_decode(model, [c.copy() for c in caches0], 4, draft, unc, 24, 1.0, 4, 4, 1)
    got0, ks0, acc0 = speculative_decode(model, [c.copy() for c in caches0], 4, draft, unc, 24, 1.0, 4, 4, 0)
    assert got1[:24] == got0[:24] == want[:24]
    assert acc1[0] == 3 and all(a == 4 for a in acc1[1:-1])       # one miss, then every block accepted
    assert len(ks1) < len(ks0)


def test_adaptive_blocks_stop_at_the_flagged_token():
    """A substituted draft token flagged as uncertain: the block ends at it, so no round spends
    rows on draft tokens behind a likely mismatch, and fewer rows are verified in all."""
    model, caches0 = _model(23)
    want = greedy_decode(model, [c.copy() for c in caches0], 6, 40)
    draft = _edit(_edit(want, "sub", 5, model.hcfg.vocab), "sub", 17, model.hcfg.vocab)
    unc = [0.1] * len(draft)
    unc[5] = unc[17] = 3.0
    got, ks, accs = speculative_decode(model, [c.copy() for c in caches0], 6, draft, unc, 32, 1.0, 2, 16, 0)
    assert got[:32] == want[:32]
    assert ks[0] == 6 and accs[0] == 5                 # ends at the flagged token, which is rejected
    fixed, ks_f, _ = speculative_decode(model, [c.copy() for c in caches0], 6, draft, [0.0] * len(draft), 32, 1.0,
                                        16, 16, 0)
    assert fixed[:32] == want[:32]
    assert sum(ks) < sum(ks_f)


def test_recycling_realigns_after_a_dropped_token():
    """A token the draft dropped: the round that misses it takes the substitution reading, the
    next one fails at once on the token the draft holds there, and the backward match puts the
    draft back in step; the substitution reading alone stays one token ahead and keeps missing."""
    model, caches0 = _model(27)
    want = greedy_decode(model, [c.copy() for c in caches0], 8, 30)
    assert len(set(want[:10])) == 10          # no repeats near the edit: every realignment is real
    draft = _edit(want, "del", 5, model.hcfg.vocab)
    unc = [0.0] * len(draft)
    got1, ks1, acc1 = speculative_decode(model, [c.copy() for c in caches0], 8, draft, unc, 24, 1.0, 4, 4, 2)
    got0, ks0, acc0 = speculative_decode(model, [c.copy() for c in caches0], 8, draft, unc, 24, 1.0, 4, 4, 0)
    assert got1[:24] == got0[:24] == want[:24]
    assert acc1[:4] == [4, 1, 0, 4]
    assert acc0[:4] == [4, 1, 0, 0] and len(ks1) < len(ks0)
