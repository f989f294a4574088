"""GPU parity of the rest of the decoder layer (post-attention RMSNorm, gated SiLU MLP,
residual) and of the whole decoder layer against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import TOL, SeededLayer, check_rounded_rows, device_cache, fill_cache, oracle_cache, rel_err, tdt, \
    to_bits, to_dev

pytestmark = pytest.mark.gpu


class SeededMlp:
    def __init__(self, stream, layer, hidden, inter, dtype):
        self.bits = si.mlp_weights(stream, layer, hidden, inter, dtype)
        self.dev = ga.MlpWeights(*(to_dev(self.bits[n], dtype) for n in ("post_norm_w", "w_gate", "w_up", "w_down")))
        self.ref = oracle.MlpWeights.from_bits(self.bits, dtype)
        self.ocfg = oracle.MlpConfig(hidden=hidden, intermediate=inter, dtype=dtype)


@pytest.mark.parametrize("dtype", [si.BF16, si.F16])
@pytest.mark.parametrize("rows,hidden,inter", [(1, 1024, 3072), (2, 1024, 3072), (4, 1024, 3072), (5, 1024, 3072),
                                               (16, 1024, 3072), (17, 1024, 3072), (64, 1024, 3072), (1, 2048, 6144),
                                               (3, 2048, 6144), (17, 2048, 6144), (64, 2048, 6144),
                                               (1, 1280, 2816), (3, 768, 1280)])
def test_mlp_vs_oracle(dtype, rows, hidden, inter):
    M = SeededMlp(30, rows, hidden, inter, dtype)
    h = si.hidden_f32(30, rows, 0, rows, hidden)
    cfg = ga.mlp_config(hidden=hidden, intermediate=inter, dtype=dtype)
    out = torch.empty((rows, hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(ga.mlp_workspace_bytes(cfg, rows), dtype=torch.uint8, device="cuda")
    ga.mlp_layer(cfg, M.dev, torch.from_numpy(h).cuda(), out, ws)
    torch.cuda.synchronize()
    want = oracle.mlp(M.ocfg, M.ref, h.astype(np.float64))
    err = rel_err(out.cpu().numpy(), want)
    # the MLP branch alone (out - h) against its own size: the residual must not hide its errors
    branch = rel_err(out.cpu().numpy().astype(np.float64) - h, want - h)
    print(f"mlp {dtype} rows={rows} H={hidden}: {err:.3e} (branch {branch:.3e})")
    assert err < TOL[dtype] and branch < TOL[dtype]


@pytest.mark.parametrize("dtype", [si.BF16, si.F16])
@pytest.mark.parametrize("rows", [9, 3])
def test_mlp_16bit_input_and_output(dtype, rows):
    hidden, inter = 1024, 3072
    M = SeededMlp(31, 0, hidden, inter, dtype)
    hb = si.activations(31, 0, 0, rows, hidden, dtype)
    cfg = ga.mlp_config(hidden=hidden, intermediate=inter, dtype=dtype, in_dtype=dtype, out_dtype=dtype)
    out = torch.empty((rows, hidden), dtype=tdt(dtype), device="cuda")
    ws = torch.empty(ga.mlp_workspace_bytes(cfg, rows), dtype=torch.uint8, device="cuda")
    ga.mlp_layer(cfg, M.dev, to_dev(hb, dtype), out, ws)
    torch.cuda.synchronize()
    want = oracle.mlp(M.ocfg, M.ref, oracle.widen(hb, dtype))
    check_rounded_rows(to_bits(out), oracle.rne16(want, dtype), dtype, rel=5e-5)


@pytest.mark.parametrize("B,lens", [(1, [795]), (6, [0, 17, 300, 64, 511, 1])])
def test_decoder_layer_decode_vs_oracle(B, lens):
    dtype = si.F16 if B == 1 else si.BF16
    cap = 832
    L = SeededLayer(32, B, 1024, dtype)
    M = SeededMlp(32, B, 1024, 3072, dtype)
    kb, vb = fill_cache(32, B, lens, cap, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = si.activations(32, B, 0, B, 1024, dtype)
    acfg, mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype)
    out = torch.empty((B, 1024), dtype=torch.float32, device="cuda")
    ws = ga.decoder_layer_workspace(acfg, mcfg, B, cap)
    ga.decoder_layer_decode(acfg, L.dev, mcfg, M.dev, kv, to_dev(xb, dtype), out, ws, host_lens=lens)
    torch.cuda.synchronize()
    want = oracle.decoder_layer_decode(L.ocfg, L.ref, M.ocfg, M.ref, ref, xb)
    err = rel_err(out.cpu().numpy(), want)
    print(f"decoder layer decode B={B} {dtype}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + 1 for l in lens]
    kg = to_bits(kv.k)
    for s in range(B):
        check_rounded_rows(kg[s, :, lens[s]], ref.k[s, :, lens[s]], dtype)


def test_decoder_layer_verify_vs_oracle():
    dtype, k = si.BF16, 4
    lens = [40, 250]
    cap = 300
    L = SeededLayer(33, 0, 1024, dtype)
    M = SeededMlp(33, 0, 1024, 3072, dtype)
    kb, vb = fill_cache(33, 0, lens, cap, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype)
    xb = si.activations(33, 0, 1, 2 * k, 1024, dtype).reshape(2, k, 1024)
    acfg, mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype)
    out = torch.empty((2, k, 1024), dtype=torch.float32, device="cuda")
    ws = ga.decoder_layer_workspace(acfg, mcfg, 2 * k, cap)
    ga.decoder_layer_verify(acfg, L.dev, mcfg, M.dev, kv, to_dev(xb, dtype), out, ws)
    torch.cuda.synchronize()
    want = oracle.decoder_layer_verify(L.ocfg, L.ref, M.ocfg, M.ref, ref, xb)
    err = rel_err(out.cpu().numpy(), want)
    print(f"decoder layer verify k={k}: {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + k for l in lens]


def test_decoder_layer_batch64_full_size_sampled():
    """64 sequences, bf16, hidden 1024 (intermediate 3072), lengths uniform in [200, 1500]: four
    sequences against the oracle, every row finite, lengths advanced."""
    dtype = si.BF16
    wl = si.WORKLOADS["ragged_batch64_h1024"]
    lens = [int(v) for v in si.kv_lengths(wl["stream"], 64, *wl["kv_len"])]
    cap = 1536
    L = SeededLayer(34, 0, 1024, dtype)
    M = SeededMlp(34, 0, 1024, 3072, dtype)
    pick = [0, 17, 42, 63]
    kb, vb = fill_cache(34, 0, lens, cap, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    xb = si.activations(34, 0, 0, 64, 1024, dtype)
    acfg, mcfg = ga.config(dtype=dtype), ga.mlp_config(dtype=dtype)
    out = torch.empty((64, 1024), dtype=torch.float32, device="cuda")
    ws = ga.decoder_layer_workspace(acfg, mcfg, 64, cap)
    ga.decoder_layer_decode(acfg, L.dev, mcfg, M.dev, kv, to_dev(xb, dtype), out, ws, host_lens=lens)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = oracle_cache(kb, vb, lens, dtype, seqs=pick)
    want = oracle.decoder_layer_decode(L.ocfg, L.ref, M.ocfg, M.ref, ref, xb[pick])
    err = rel_err(got[pick], want)
    print(f"decoder layer batch 64 (4 sampled): {err:.3e}")
    assert err < TOL[dtype]
    assert kv.lens.cpu().tolist() == [l + 1 for l in lens]
