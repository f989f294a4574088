"""GPU parity of batched speculative decoding with per-sequence block lengths ("Can CTC make
Qwen3-ASR faster?", section 07 and section 08 "Verifier, version 0"): every round embeds one
block per sequence, runs the mixed decoder layers over all of them at once, takes the argmax of
every row, accepts per sequence and crops; the host picks each sequence's next block length from
its draft's uncertainties and recycles its draft after a correction.  The committed transcripts,
block lengths and accepted counts equal the oracle's for every sequence."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import SeededLayer, tdt, to_dev

pytestmark = pytest.mark.gpu


class BatchModel:
    """Two decoder layers at the 0.6B shapes with a 2,048-id vocabulary for B sequences, each
    with its own prompt in its cache slot; the oracle model and one oracle cache per sequence."""

    def __init__(self, stream, prompts, dtype=si.BF16, n_layers=2, V=2048, cap=128):
        H, I = 1024, 3072
        B = len(prompts)
        self.dtype, self.V, self.H, self.B = dtype, V, H, B
        self.acfg, self.mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype, out_dtype=dtype)
        self.mcfg_last = ga.mlp_config(dtype=dtype)
        self.hcfg = ga.head_config(hidden=H, vocab=V, dtype=dtype)
        hb = si.head_weights(stream, H, V, dtype)
        self.attn = [SeededLayer(stream, l, H, dtype) for l in range(n_layers)]
        mlpb = [si.mlp_weights(stream, l, H, I, dtype) for l in range(n_layers)]
        self.mlp = [ga.MlpWeights(*(to_dev(b[n], dtype) for n in ("post_norm_w", "w_gate", "w_up", "w_down")))
                    for b in mlpb]
        self.table = to_dev(hb["embed"], dtype)
        self.gfin, self.wlm = to_dev(hb["final_norm_w"], dtype), to_dev(hb["w_lm"], dtype)
        self.kvs = [ga.KVLayer.empty(B, 8, cap, dtype=tdt(dtype)) for _ in range(n_layers)]
        self.ocaches = [[] for _ in range(B)]
        for l in range(n_layers):
            for s, P in enumerate(prompts):
                kb, vb = si.kv_rows(stream, l, s, P, dtype)
                self.kvs[l].k[s, :, :P], self.kvs[l].v[s, :, :P] = to_dev(kb, dtype), to_dev(vb, dtype)
                c = oracle.KVCache.empty(1, 8, cap, 128, dtype)
                c.k[0, :, :P], c.v[0, :, :P], c.lens[0] = kb, vb, P
                self.ocaches[s].append(c)
            self.kvs[l].lens.copy_(torch.tensor(prompts, dtype=torch.int32))
        self.ref = oracle.TinyModel(self.attn[0].ocfg, oracle.MlpConfig(hidden=H, intermediate=I, dtype=dtype),
                                    oracle.HeadConfig(hidden=H, vocab=V, dtype=dtype), hb["embed"],
                                    [(a.ref, oracle.MlpWeights.from_bits(m, dtype)) for a, m in zip(self.attn, mlpb)],
                                    oracle.widen(hb["final_norm_w"], dtype), oracle.widen(hb["w_lm"], dtype))
        self.ws = ga.decoder_layer_workspace(self.acfg, self.mcfg, 16 * B, cap)
        self.hws = ga.lm_head_workspace(self.hcfg, 16 * B)


def _edit(seq, kind, at, vocab):
    s = list(seq)
    if kind == "sub":
        s[at] = (s[at] + 1) % vocab
    elif kind == "ins":
        s.insert(at, (s[at] + 7) % vocab)
    elif kind == "del":
        del s[at]
    return s


def test_mixed_acceptance_is_bit_exact():
    """Packed blocks of sizes 1 .. 16 with mismatches anywhere (or none): accepted counts, next
    tokens and crop lengths equal the oracle's rule per sequence."""
    g = np.random.default_rng(48)
    sizes = [1, 5, 16, 3, 8, 2, 1, 11]
    B, cap = len(sizes), 12
    slots = g.permutation(cap)[:B].astype(np.int32)
    draft, target = [], []
    for k in sizes:
        d = g.integers(0, 9, k)
        t = d.copy()
        a = int(g.integers(0, k + 1))
        if a < k:
            t[a] = (d[a] + 1 + int(g.integers(0, 3))) % 9
            t[a + 1:] = g.integers(0, 9, k - a - 1)
        draft += d.tolist()
        target += t.tolist()
    lens = g.integers(16, 60, cap).astype(np.int32)
    dv = lambda a: torch.tensor(np.asarray(a, np.int32), device="cuda")
    acc, nxt, nl = (torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda"),
                    torch.empty(cap, dtype=torch.int32, device="cuda"))
    ga.accept_greedy_mixed(dv(draft), dv(target), sizes, dv(lens), acc, nxt, nl, slots=dv(slots))
    torch.cuda.synchronize()
    want = lens.copy()
    r = 0
    for b, k in enumerate(sizes):
        a, corr, committed = oracle.accept_greedy(draft[r:r + k], target[r:r + k])
        assert acc[b].item() == a
        assert nxt[b].item() == (corr if corr is not None else draft[r + k - 1])
        want[slots[b]] = lens[slots[b]] - k + committed
        r += k
    assert np.array_equal(nl.cpu().numpy(), want)


@pytest.mark.parametrize("window,k_min,k_max", [(2, 2, 8), (0, 4, 4), (4, 1, 16)])
def test_batched_speculative_decoding_with_adaptive_blocks_and_recycling(window, k_min, k_max):
    prompts = [20, 33, 7, 51]
    first = [9, 100, 1500, 3]
    edits = [[("sub", 3)], [("ins", 2), ("sub", 9)], [], [("del", 5), ("ins", 12)]]
    n_tok, tau = 16, 1.0
    m = BatchModel(47, prompts)
    B = len(prompts)
    # the oracle: greedy transcripts, the drafts built from them, and the speculative decodes
    drafts, uncs, want = [], [], []
    for s in range(B):
        greedy = oracle.greedy_decode(m.ref, [c.copy() for c in m.ocaches[s]], first[s], n_tok + 8)
        d = greedy
        for kind, at in edits[s][::-1]:
            d = _edit(d, kind, at, m.V)
        u = [0.2] * len(d)
        for kind, at in edits[s]:
            u[min(at, len(d) - 1)] = 3.0
        drafts.append(d)
        uncs.append(u)
        got, ks, accs = oracle.speculative_decode(m.ref, [c.copy() for c in m.ocaches[s]], first[s], d, u, n_tok,
                                                  tau, k_min, k_max, window)
        assert got[:n_tok] == greedy[:n_tok]
        want.append((got, ks, accs))
    # the device, all sequences in one mixed batch per round
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    new_lens = torch.empty(B, dtype=torch.int32, device="cuda")
    pos, last = [0] * B, list(first)
    got = [[] for _ in range(B)]
    ks = [[] for _ in range(B)]
    accs = [[] for _ in range(B)]
    done = [False] * B
    while not all(done):
        act = [s for s in range(B) if not done[s]]
        kk = [ga.next_block_len(uncs[s][pos[s]:], tau, k_min, k_max) for s in act]
        dr = [(drafts[s][pos[s]:] + [-1] * k)[:k] for s, k in zip(act, kk)]
        blocks = [[last[s]] + d[:k - 1] for s, d, k in zip(act, dr, kk)]
        # sequences that are done sit this round out: the mixed call takes the active slots
        sizes = kk
        rows = sum(sizes)
        ids = torch.tensor([t for b in blocks for t in b], dtype=torch.int32, device="cuda")
        x = torch.empty((rows, m.H), dtype=tdt(m.dtype), device="cuda")
        ga.embed(m.table, ids, x)
        slots = torch.tensor(act, dtype=torch.int32, device="cuda")
        for l, (a, mw, kv) in enumerate(zip(m.attn, m.mlp, m.kvs)):
            lastl = l == len(m.kvs) - 1
            out = torch.empty((rows, m.H), dtype=torch.float32 if lastl else tdt(m.dtype), device="cuda")
            ga.decoder_layer_mixed(m.acfg, a.dev, m.mcfg_last if lastl else m.mcfg, mw, kv, x, sizes, out, m.ws,
                                   slots=slots)
            x = out
        tgt = torch.empty(rows, dtype=torch.int32, device="cuda")
        ga.lm_head_argmax(m.hcfg, m.gfin, m.wlm, x, tgt, m.hws)
        dflat = torch.tensor([t for d in dr for t in d], dtype=torch.int32, device="cuda")
        ga.accept_greedy_mixed(dflat, tgt, sizes, m.kvs[0].lens, acc[:len(act)], nxt[:len(act)], new_lens,
                               slots=slots)
        ga.kv_crop(m.kvs, new_lens)
        A, N = acc[:len(act)].cpu().tolist(), nxt[:len(act)].cpu().tolist()
        for i, s in enumerate(act):
            k, a = kk[i], A[i]
            committed = dr[i][:a] + ([] if a == k else [N[i]])
            pos[s] = ga.recycle_draft(drafts[s], pos[s], k, a, None if a == k else N[i], window)
            got[s] += committed
            ks[s].append(k)
            accs[s].append(a)
            last[s] = got[s][-1]
            done[s] = len(got[s]) >= n_tok
    lens = m.kvs[0].lens.cpu().tolist()
    for s in range(B):
        print(f"seq {s}: blocks {ks[s]} accepted {accs[s]}")
        assert got[s] == want[s][0]
        assert ks[s] == want[s][1] and accs[s] == want[s][2]
        assert lens[s] == prompts[s] + len(got[s])
