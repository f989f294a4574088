"""Parity at the five workloads' full sizes, in the launch configuration the benchmark times.

Layers are independent (each has its own weights, cache and inputs), so a
sample of layers is run with exactly the per-layer launch of the 28-layer
stack; the oracle checks every output of the sampled layers (bs1) or the
outputs of sampled sequences (batch 64).
"""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import TOL, SeededLayer, device_cache, fill_cache, oracle_cache, rel_err, to_bits, to_dev, check_rounded_rows

pytestmark = pytest.mark.gpu

CAPACITY = {"decode_bs1_1layer_kv64": 128, "decode_bs1_28layers_kv795": 928, "verify_bs1_28layers_kv795": 832,
            "ragged_batch64_h1024": 1536, "ragged_batch64_h2048": 4112}   # the benchmark's cache capacities
SAMPLE_LAYERS = (0, 27)


def test_decode_bs1_28layers_130_steps_sampled_layers():
    """bs1, fp16: prefill 795, then 130 decode steps (KV 795 -> 925); every step checked."""
    name = "decode_bs1_28layers_kv795"
    c = si.WORKLOADS[name]
    dtype, H, cap, sid = c["dtype"], c["hidden"], CAPACITY[name], c["stream"]
    cfg = ga.config(dtype=dtype)
    ws = ga.alloc_workspace(cfg, 1, cap)
    worst = 0.0
    for layer in SAMPLE_LAYERS:
        L = SeededLayer(sid, layer, H, dtype)
        kb, vb = fill_cache(sid, layer, [795], cap, dtype)
        kv = device_cache(kb, vb, [795], dtype)
        ref = oracle_cache(kb, vb, [795], dtype)
        xs = np.stack([si.activations(sid, layer, s, 1, H, dtype) for s in range(130)])
        xdev = to_dev(xs, dtype)
        outs = torch.empty((130, 1, H), dtype=torch.float32, device="cuda")
        for s in range(130):
            ga.layer_decode(cfg, L.dev, kv, xdev[s], outs[s], ws, host_lens=[795 + s])
        torch.cuda.synchronize()
        got = outs.cpu().numpy().astype(np.float64)
        for s in range(130):
            want = oracle.decode(L.ocfg, L.ref, ref, xs[s])
            worst = max(worst, rel_err(got[s], want))
        assert kv.lens.item() == 925
        check_rounded_rows(to_bits(kv.k)[0, :, 795:925], ref.k[0, :, 795:925], dtype)
    print(f"bs1 decode worst max|err|/rms over 2 layers x 130 steps = {worst:.3e}")
    assert worst < TOL[dtype]


@pytest.mark.parametrize("k", [4, 8, 16])
def test_verify_bs1_kv795_crop_then_decode(k):
    name = "verify_bs1_28layers_kv795"
    c = si.WORKLOADS[name]
    dtype, H, cap, sid = c["dtype"], c["hidden"], CAPACITY[name], c["stream"]
    cfg = ga.config(dtype=dtype)
    worst = 0.0
    for layer in SAMPLE_LAYERS:
        L = SeededLayer(sid, layer, H, dtype)
        kb, vb = fill_cache(sid, layer, [795], cap, dtype)
        kv = device_cache(kb, vb, [795], dtype)
        ref = oracle_cache(kb, vb, [795], dtype)
        xs = si.activations(sid, layer, k, k, H, dtype).reshape(1, k, H)
        ws = ga.alloc_workspace(cfg, k, cap)
        out = torch.empty((1, k, H), dtype=torch.float32, device="cuda")
        ga.layer_verify(cfg, L.dev, kv, to_dev(xs, dtype), out, ws, host_lens=[795])
        want = oracle.verify(L.ocfg, L.ref, ref, xs)
        torch.cuda.synchronize()
        worst = max(worst, rel_err(out.cpu().numpy(), want))
        a = si.accepted_prefix(sid, k)
        ga.kv_crop([kv], torch.tensor([795 + a], dtype=torch.int32, device="cuda"))
        oracle.kv_crop([ref], [795 + a])
        xn = si.activations(sid, layer, 100 + k, 1, H, dtype)
        o2 = torch.empty((1, H), dtype=torch.float32, device="cuda")
        ga.layer_decode(cfg, L.dev, kv, to_dev(xn, dtype), o2, ws, host_lens=[795 + a])
        want2 = oracle.decode(L.ocfg, L.ref, ref, xn)
        torch.cuda.synchronize()
        worst = max(worst, rel_err(o2.cpu().numpy(), want2))
        assert kv.lens.item() == 795 + a + 1 and kv.status.item() == 0
    print(f"bs1 verify k={k} worst = {worst:.3e}")
    assert worst < TOL[dtype]


def _batched(name, layer, verify_after=False):
    c = si.WORKLOADS[name]
    dtype, H, B, cap, stream = c["dtype"], c["hidden"], c["batch"], CAPACITY[name], c["stream"]
    lens = si.kv_lengths(stream, B, *c["kv_len"])
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5, 17, 40})
    L = SeededLayer(stream, layer, H, dtype)
    kb, vb = fill_cache(stream, layer, lens, cap, dtype)
    kv = device_cache(kb, vb, lens, dtype)
    ref = oracle_cache(kb, vb, lens, dtype, seqs=pick)
    cfg = ga.config(hidden=H, dtype=dtype)
    xs = si.activations(stream, layer, 0, B, H, dtype)
    ws = ga.alloc_workspace(cfg, B, cap)
    out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ga.layer_decode(cfg, L.dev, kv, to_dev(xs, dtype), out, ws, host_lens=lens.tolist())
    torch.cuda.synchronize()
    want = oracle.decode(L.ocfg, L.ref, ref, xs[pick])
    err = rel_err(out.cpu().numpy()[pick], want)
    assert kv.lens.cpu().numpy().tolist() == (lens + 1).tolist()
    kg = to_bits(kv.k)[pick]
    idx = np.arange(len(pick))
    check_rounded_rows(kg[idx, :, lens[pick]], ref.k[idx, :, lens[pick]], dtype)
    if verify_after:
        k, nseq = c["verify_k"][0], c["verify_seqs"]
        chosen = si.verify_choice(stream, B, nseq)
        xv = si.activations(stream, layer, 1, nseq * k, H, dtype).reshape(nseq, k, H)
        wsv = ga.alloc_workspace(cfg, nseq * k, cap)
        outv = torch.empty((nseq, k, H), dtype=torch.float32, device="cuda")
        ga.layer_verify(cfg, L.dev, kv, to_dev(xv, dtype), outv, wsv,
                        slots=torch.tensor(chosen, dtype=torch.int32, device="cuda"),
                        host_lens=(lens[chosen] + 1).tolist())
        torch.cuda.synchronize()
        vpick = [0, nseq - 1]
        seqs = [int(chosen[i]) for i in vpick]
        refv = oracle_cache(kb, vb, lens, dtype, seqs=seqs)
        # replay the decode step on these sequences first (their caches grew by one row)
        oracle.decode(L.ocfg, L.ref, refv, xs[seqs])
        wantv = oracle.verify(L.ocfg, L.ref, refv, xv[vpick])
        err = max(err, rel_err(outv.cpu().numpy()[vpick], wantv))
        got_lens = kv.lens.cpu().numpy()
        assert np.all(got_lens[chosen] == lens[chosen] + 1 + k)
    return err


@pytest.mark.parametrize("layer", SAMPLE_LAYERS)
def test_ragged_batch64_h1024_decode(layer):
    err = _batched("ragged_batch64_h1024", layer)
    print(f"batch 64, hidden 1024, layer {layer}: {err:.3e}")
    assert err < TOL[si.BF16]


@pytest.mark.parametrize("layer", SAMPLE_LAYERS)
def test_ragged_batch64_h2048_decode_and_verify(layer):
    err = _batched("ragged_batch64_h2048", layer, verify_after=True)
    print(f"batch 64, hidden 2048, layer {layer}: {err:.3e}")
    assert err < TOL[si.BF16]
