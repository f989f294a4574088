"""GPU parity of the verify loop: embedding, lm_head argmax, greedy acceptance, and whole
speculative rounds on a two-layer model committing exactly the greedy transcript ("Can CTC
make Qwen3-ASR faster?", section 03 "Greedy exactness", section 11 Phase A)."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import SeededLayer, tdt, to_bits, to_dev

pytestmark = pytest.mark.gpu


def test_embed_rows_and_out_of_range_ids():
    dtype = si.BF16
    hb = si.head_weights(40, 1024, 512, dtype)
    table = to_dev(hb["embed"], dtype)
    ids = [3, 511, 0, 512, -1, 77]
    x = torch.empty((6, 1024), dtype=tdt(dtype), device="cuda")
    ga.embed(table, torch.tensor(ids, dtype=torch.int32, device="cuda"), x)
    torch.cuda.synchronize()
    got = to_bits(x)
    for r, i in enumerate(ids):
        if 0 <= i < 512:
            assert np.array_equal(got[r], oracle.embed(hb["embed"], [i])[0])
        else:
            assert np.all(np.isnan(oracle.widen(got[r], dtype)))


def _head_check(got_ids, got_max, logits, scale):
    """The GPU's id must be an argmax of the oracle's logits up to the fp32 error of a logit, and
    equal to the oracle's where the top two are further apart than that."""
    eps = 1e-4 * scale
    top = np.max(logits, axis=1)
    srt = np.sort(logits, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    for r in range(len(got_ids)):
        assert 0 <= got_ids[r] < logits.shape[1]
        assert logits[r, got_ids[r]] >= top[r] - eps
        assert abs(got_max[r] - top[r]) <= eps
        if gap[r] > 2 * eps:
            assert got_ids[r] == int(np.argmax(logits[r]))
    return int(np.sum(gap > 2 * eps))


@pytest.mark.parametrize("rows", [1, 9, 17])
def test_lm_head_argmax_full_vocab_vs_oracle(rows):
    """The Qwen3 vocabulary (151,936 ids) at hidden 1024, fp32 rows in."""
    dtype, H, V = si.BF16, 1024, 151936
    hb = si.head_weights(41, H, V, dtype)
    h = si.hidden_f32(41, 0, rows, rows, H)
    cfg = ga.head_config(hidden=H, vocab=V, dtype=dtype)
    ids = torch.empty(rows, dtype=torch.int32, device="cuda")
    mx = torch.empty(rows, dtype=torch.float32, device="cuda")
    ga.lm_head_argmax(cfg, to_dev(hb["final_norm_w"], dtype), to_dev(hb["w_lm"], dtype), torch.from_numpy(h).cuda(),
                      ids, ga.lm_head_workspace(cfg, rows), max_logit=mx)
    torch.cuda.synchronize()
    logits = oracle.lm_head_logits(oracle.HeadConfig(hidden=H, vocab=V), oracle.widen(hb["final_norm_w"], dtype),
                                   oracle.widen(hb["w_lm"], dtype), h.astype(np.float64))
    n = _head_check(ids.cpu().numpy(), mx.cpu().numpy(), logits, float(np.sqrt(np.mean(logits ** 2))))
    print(f"lm_head argmax rows={rows}: {n}/{rows} rows with a unique argmax, all equal")


def test_lm_head_argmax_16bit_rows_and_ties():
    """16-bit rows in; rows whose logits tie exactly (duplicated lm_head rows) take the smaller id."""
    dtype, H, V = si.F16, 1024, 4096
    hb = si.head_weights(42, H, V, dtype)
    w = hb["w_lm"].copy()
    hx = si.activations(42, 0, 0, 6, H, dtype)
    logits = oracle.lm_head_logits(oracle.HeadConfig(hidden=H, vocab=V), oracle.widen(hb["final_norm_w"], dtype),
                                   oracle.widen(w, dtype), oracle.widen(hx, dtype))
    best = np.argmax(logits, axis=1)
    for r in range(6):   # copy each row's winning lm_head row to a larger id: an exact tie
        w[(best[r] + 1000) % V] = w[best[r]] if (best[r] + 1000) % V > best[r] else w[(best[r] + 1000) % V]
    cfg = ga.head_config(hidden=H, vocab=V, dtype=dtype, in_dtype=dtype)
    ids = torch.empty(6, dtype=torch.int32, device="cuda")
    mx = torch.empty(6, dtype=torch.float32, device="cuda")
    ga.lm_head_argmax(cfg, to_dev(hb["final_norm_w"], dtype), to_dev(w, dtype), to_dev(hx, dtype), ids,
                      ga.lm_head_workspace(cfg, 6), max_logit=mx)
    torch.cuda.synchronize()
    logits = oracle.lm_head_logits(oracle.HeadConfig(hidden=H, vocab=V), oracle.widen(hb["final_norm_w"], dtype),
                                   oracle.widen(w, dtype), oracle.widen(hx, dtype))
    _head_check(ids.cpu().numpy(), mx.cpu().numpy(), logits, float(np.sqrt(np.mean(logits ** 2))))
    assert np.array_equal(ids.cpu().numpy(), oracle.argmax_first(logits))


@pytest.mark.parametrize("k", [1, 3, 8])
def test_accept_greedy_is_bit_exact(k):
    g = np.random.default_rng(k)
    B, cap = 37, 50
    slots = g.permutation(cap)[:B].astype(np.int32)
    draft = g.integers(0, 6, (B, k)).astype(np.int32)
    target = draft.copy()
    for b in range(B):     # a mismatch at a random place, or none
        a = int(g.integers(0, k + 1))
        if a < k:
            target[b, a] = (draft[b, a] + 1 + int(g.integers(0, 3))) % 9
        target[b, a + 1:] = g.integers(0, 6, k - a - 1) if a + 1 < k else target[b, a + 1:]
    lens = g.integers(k, 40, cap).astype(np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    acc, nxt, nl = (torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda"),
                    torch.empty(cap, dtype=torch.int32, device="cuda"))
    ga.accept_greedy(d(draft), d(target), d(lens), acc, nxt, nl, slots=d(slots))
    torch.cuda.synchronize()
    want_lens = lens.copy()
    for b in range(B):
        a, corr, committed = oracle.accept_greedy(draft[b].tolist(), target[b].tolist())
        assert acc[b].item() == a
        assert nxt[b].item() == (corr if corr is not None else draft[b, -1])
        want_lens[slots[b]] = lens[slots[b]] - k + committed
    assert np.array_equal(nl.cpu().numpy(), want_lens)


class TinyGpuModel:
    """Two decoder layers at the 0.6B shapes (hidden 1024, 16 q / 8 kv heads, intermediate 3072)
    with a 2,048-id vocabulary, on the device and in the oracle; a 20-position prompt in every
    layer's cache."""

    def __init__(self, stream, dtype=si.BF16, n_layers=2, V=2048, prompt=20, cap=96):
        H, I = 1024, 3072
        self.dtype, self.V, self.H = dtype, V, H
        self.acfg, self.mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype, out_dtype=dtype)
        self.mcfg_last = ga.mlp_config(dtype=dtype)
        self.hcfg = ga.head_config(hidden=H, vocab=V, dtype=dtype)
        hb = si.head_weights(stream, H, V, dtype)
        self.attn = [SeededLayer(stream, l, H, dtype) for l in range(n_layers)]
        self.mlpb = [si.mlp_weights(stream, l, H, I, dtype) for l in range(n_layers)]
        self.mlp = [ga.MlpWeights(*(to_dev(b[n], dtype) for n in ("post_norm_w", "w_gate", "w_up", "w_down")))
                    for b in self.mlpb]
        self.table = to_dev(hb["embed"], dtype)
        self.gfin, self.wlm = to_dev(hb["final_norm_w"], dtype), to_dev(hb["w_lm"], dtype)
        self.kvs, ocaches = [], []
        for l in range(n_layers):
            kb, vb = si.kv_rows(stream, l, 0, prompt, dtype)
            kv = ga.KVLayer.empty(1, 8, cap, dtype=tdt(dtype))
            kv.k[0, :, :prompt], kv.v[0, :, :prompt] = to_dev(kb, dtype), to_dev(vb, dtype)
            kv.lens.fill_(prompt)
            self.kvs.append(kv)
            c = oracle.KVCache.empty(1, 8, cap, 128, dtype)
            c.k[0, :, :prompt], c.v[0, :, :prompt], c.lens[0] = kb, vb, prompt
            ocaches.append(c)
        self.ref = oracle.TinyModel(self.attn[0].ocfg, oracle.MlpConfig(hidden=H, intermediate=I, dtype=dtype),
                                    oracle.HeadConfig(hidden=H, vocab=V, dtype=dtype), hb["embed"],
                                    [(a.ref, oracle.MlpWeights.from_bits(m, dtype)) for a, m in zip(self.attn, self.mlpb)],
                                    oracle.widen(hb["final_norm_w"], dtype), oracle.widen(hb["w_lm"], dtype))
        self.ocaches = ocaches
        self.ws = ga.decoder_layer_workspace(self.acfg, self.mcfg, 16, cap)
        self.hws = ga.lm_head_workspace(self.hcfg, 16)

    def forward(self, tokens):
        """The block of tokens through every layer and the head: argmax id of every row."""
        n = len(tokens)
        ids = torch.tensor(tokens, dtype=torch.int32, device="cuda")
        x = torch.empty((n, self.H), dtype=tdt(self.dtype), device="cuda")
        ga.embed(self.table, ids, x)
        for l, (a, m, kv) in enumerate(zip(self.attn, self.mlp, self.kvs)):
            last = l == len(self.kvs) - 1
            out = torch.empty((n, self.H), dtype=torch.float32 if last else tdt(self.dtype), device="cuda")
            mcfg = self.mcfg_last if last else self.mcfg
            if n == 1:
                ga.decoder_layer_decode(self.acfg, a.dev, mcfg, m, kv, x, out, self.ws)
            else:
                ga.decoder_layer_verify(self.acfg, a.dev, mcfg, m, kv, x.view(1, n, self.H), out.view(1, n, self.H),
                                        self.ws)
            x = out
        am = torch.empty(n, dtype=torch.int32, device="cuda")
        ga.lm_head_argmax(self.hcfg, self.gfin, self.wlm, x, am, self.hws)
        return am


def test_gpu_greedy_decode_matches_the_oracle_model():
    m = TinyGpuModel(43)
    gpu, tok = [], 7
    for _ in range(8):
        tok = int(m.forward([tok]).cpu()[0])
        gpu.append(tok)
    want = oracle.greedy_decode(m.ref, m.ocaches, 7, 8)
    print(f"greedy: gpu {gpu} oracle {want}")
    assert gpu == want


@pytest.mark.parametrize("bad", [None, 0, 2])
def test_gpu_speculative_rounds_commit_the_greedy_transcript(bad):
    """Greedy decoding on the GPU, then speculative rounds of k = 4 on a fresh copy with the
    greedy transcript as the draft (all accepted) or wrong at position `bad` of every round:
    embedding, two verify layers, lm_head argmax, acceptance and crop, all on the device; the
    committed transcript equals the greedy one and every layer keeps exactly its tokens."""
    k, n_tok = 4, 12
    ref = TinyGpuModel(44)
    greedy, tok = [], 9
    for _ in range(n_tok):
        tok = int(ref.forward([tok]).cpu()[0])
        greedy.append(tok)
    m = TinyGpuModel(44)
    got, last = [], 9
    acc = torch.empty(1, dtype=torch.int32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    new_lens = torch.empty(1, dtype=torch.int32, device="cuda")
    while len(got) < n_tok:
        draft = (greedy[len(got):] + [0] * k)[:k]
        if bad is not None:
            draft[bad] = (draft[bad] + 1) % m.V
        target = m.forward([last] + draft[:k - 1])
        ga.accept_greedy(torch.tensor([draft], dtype=torch.int32, device="cuda"), target.view(1, k),
                         m.kvs[0].lens, acc, nxt, new_lens)
        ga.kv_crop(m.kvs, new_lens)
        a = int(acc.item())
        got += draft[:a] + ([] if a == k else [int(nxt.item())])
        last = got[-1]
        if bad is None and len(got) < n_tok:
            assert a == k
    assert got[:n_tok] == greedy
    assert all(int(kv.lens.item()) == 20 + len(got) for kv in m.kvs)
