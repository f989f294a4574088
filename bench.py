#!/usr/bin/env python3
"""Benchmark of the decoder attention block on one MI355X.

Headline workload: the 28-layer attention stack of Qwen3-ASR-0.6B decoding
at batch 1 in fp16 (hidden 1024, 16 q / 8 kv heads, head_dim 128), with a
795-token prefilled cache and 130 generated tokens (KV 795 -> 925): the clip
of "Qwen3-ASR -- Latency & Bottleneck Analysis", section 01.  One step = one
generated token = 28 layer calls; step s of a 130-step round uses cache
length 795 + s, and a crop returns the caches to 795 after step 129.  Each
step is one captured HIP graph, replayed, so host overhead stays out of the
timed region (the static one-token step of that page's section 08, step 2).

Second workload (``--no-batched`` skips it): ragged batched decode of 64
sequences in bf16, committed lengths uniform in [200, 1500]; one step = 28
layer calls + the crop back to the committed lengths, reported in tokens/s.
Also reported: the bs1 verify block for k = 4, 8, 16 (``--no-verify``) and
the hidden-2048 batch-64 decode with a k = 8 verify on 8 sequences
(``--no-wide``).

Roofline: a second timed region replays the same calls eagerly with HIP
events that the library has the runtime stamp at the start and end of each
phase kernel on the launch stream (hipExtLaunchKernelGGL), which gives each
kernel's average duration; the dominant kernel's algorithmic bytes over that
duration, against the 8 TB/s HBM peak, is the roofline fraction.  ``traffic``
is the counter-measured HBM bytes of that kernel per launch, reported while
the kernel sources are the ones the counters were taken on.

Prints ONE JSON line.  ``value`` = microseconds per generated token of the
28-layer block at batch 1 (lower is better).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CAP_BS1 = 928                  # cache capacity of the bs1 workload (>= 925, multiple of 16)
CAP_B64 = 1536                 # cache capacity of the batch-64 workload (>= 1501)
CAP_W64 = 4112                 # cache capacity of the hidden-2048 batch-64 workload (>= 4096 + 1 + 8)
PHASES = ("qkv_projection", "attention", "o_proj")
# the pages' figure for the same workload on another machine (context, not a target): 28 decoder
# attention layers at bs1 over the 795 -> 925 clip, RTX 3050 Laptop, HF eager, in us per token
PAGES_US_PER_TOKEN = 9033.0
# HBM bytes per launch of each phase kernel from the FETCH_SIZE and WRITE_SIZE counters, each
# scaled by what that counter reads for a 1 GiB device copy (fetch x1.99994, write x1.000), and
# the digest of the kernel sources they were taken on: reported only while the sources match
TRAFFIC = {
    "sources_sha256": "86b4dc98ed0c9ee0282ed4551f3c80a463875caaa6a1570833e4c8467d5b1b77",
    "bs1": {"qkv_projection": 8583097, "attention": 4048563, "o_proj": 4862001},
    "b64": {"qkv_projection": 11077731, "attention": 230242802, "o_proj": 8722569},
}
KERNEL_SOURCES = ("gqa_decode_attention_amd/csrc/attn_layer.hip", "gqa_decode_attention_amd/csrc/device_common.h",
                  "gqa_decode_attention_amd/csrc/internal.h", "gqa_decode_attention_amd/csrc/api.hip",
                  "gqa_decode_attention_amd/build.py")


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    return TRAFFIC[workload] if sources_digest() == TRAFFIC["sources_sha256"] else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=130)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-batched", action="store_true", help="skip the batch-64 workloads")
    p.add_argument("--no-verify", action="store_true", help="skip the bs1 verify blocks")
    p.add_argument("--no-wide", action="store_true", help="skip the hidden-2048 batch-64 workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    p.add_argument("--dispatch", type=int, default=0, help="0 auto, 1 one kernel per phase, 2 fused")
    p.add_argument("--kv-split", type=int, default=0, help="keys per split-KV chunk (0: automatic)")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="run only this many bs1 steps eagerly (for profilers) and exit")
    p.add_argument("--profile-batched", type=int, default=0,
                   help="run only this many batch-64 steps eagerly (for profilers) and exit")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run three device-to-device copies of this many MiB (counter calibration)")
    return p.parse_args()


def phase_bytes(H, nq, nkv, d, committed, rows, e_in=2, e_out=4):
    """Algorithmic HBM bytes of each phase of one layer call (workspace traffic not counted).

    qkv_projection: W_qkv, the three norm gains and x, read once.  attention: the committed K/V
    rows read once and the appended K/V rows written.  o_proj: W_o read once, out written."""
    qkv = ((nq + 2 * nkv) * d * H + H + 2 * d) * 2 + rows * H * e_in
    att = sum(committed) * 2 * nkv * d * 2 + rows * 2 * nkv * d * 2
    oproj = H * nq * d * 2 + rows * H * e_out
    return {"qkv_projection": qkv, "attention": att, "o_proj": oproj}


def layer_bytes(H, nq, nkv, d, committed, rows, e_in=2, e_out=4):
    return sum(phase_bytes(H, nq, nkv, d, committed, rows, e_in, e_out).values())


def roofline(mean_us, bphase, traffic):
    dom = max(PHASES, key=lambda k: mean_us[k])
    achieved = bphase[dom] / (mean_us[dom] * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic.get(dom) if traffic else None,
            "bytes_per_launch": round(bphase[dom]), "us_per_launch": round(mean_us[dom], 3),
            "phase_us": {k: round(v, 3) for k, v in mean_us.items()},
            "phase_bytes": {k: round(v) for k, v in bphase.items()}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(every sequence's work is independent: see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_mib:
        src = torch.ones(args.copy_mib << 19, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "bytes_read": src.numel() * 2,
                          "bytes_written": dst.numel() * 2}))
        return

    import gqa_decode_attention_amd as ga
    from synth import inputs as si

    def to_dev(bits, dtype):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.float16 if dtype == si.F16 else torch.bfloat16).to(dev)

    if args.profile_batched:
        batched_leg(args, ga, si, np, torch, dev, to_dev, stream)
        print(json.dumps({"profile_batched": args.profile_batched}))
        return

    # ------------------------------------------------------------ bs1 workload
    wl = si.WORKLOADS["decode_bs1_28layers_kv795"]
    H, NL, dtype, sid = wl["hidden"], wl["layers"], wl["dtype"], wl["stream"]
    P0, NSTEP = 795, 130
    cfg = ga.config(hidden=H, dtype=dtype, dispatch=args.dispatch, kv_split=args.kv_split)
    t0 = time.time()
    weights, kvs = [], []
    for l in range(NL):
        wb = si.layer_weights(sid, l, H, dtype)
        weights.append(ga.Weights(*(to_dev(wb[n], dtype) for n in
                                    ("input_norm_w", "w_qkv", "q_norm_w", "k_norm_w", "w_o"))))
        kb, vb = si.kv_rows(sid, l, 0, P0, dtype)
        kv = ga.KVLayer.empty(1, 8, CAP_BS1, dtype=torch.float16, device=dev)
        ga.kv_append(kv, to_dev(kb.transpose(1, 0, 2)[None], dtype), to_dev(vb.transpose(1, 0, 2)[None], dtype))
        kvs.append(kv)
    xs = torch.stack([torch.stack([to_dev(si.activations(sid, l, s, 1, H, dtype), dtype) for l in range(NL)])
                      for s in range(NSTEP)])                      # [step][layer][1][H]
    outs = torch.empty((NL, 1, H), dtype=torch.float32, device=dev)
    ws = ga.alloc_workspace(cfg, 1, CAP_BS1, device=dev)
    base_lens = torch.full((1,), P0, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] bs1 inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def step_calls(s):
        for l in range(NL):
            ga.layer_decode(cfg, weights[l], kvs[l], xs[s, l], outs[l], ws, host_lens=[P0 + s])

    if args.profile_steps:
        for s in range(args.profile_steps):
            step_calls(s % NSTEP)
            if s % NSTEP == NSTEP - 1:
                ga.kv_crop(kvs, base_lens)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps}))
        return

    graphs = []
    for s in range(NSTEP):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_calls(s)
        graphs.append(g)
    crop_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(crop_graph):
        ga.kv_crop(kvs, base_lens)
    ga.kv_crop(kvs, base_lens)        # capture only records: reset what eager work touched
    torch.cuda.synchronize()

    def run_steps(n):
        for i in range(n):
            s = i % NSTEP
            graphs[s].replay()
            if s == NSTEP - 1:
                crop_graph.replay()

    run_steps(args.warmup)
    crop_graph.replay()               # the timed region starts a round at step 0
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    run_steps(args.steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    us_token = ms_step * 1000.0
    committed = [P0 + (i % NSTEP) for i in range(args.steps)]
    bytes_call = float(np.mean([layer_bytes(H, 16, 8, 128, [L], 1) for L in committed]))
    us_call = us_token / NL
    lens_ok = all(int(kv.lens.item()) == P0 + (args.steps % NSTEP) for kv in kvs)
    status_ok = all(int(kv.status.item()) == 0 for kv in kvs)
    print(f"[bench] bs1: {us_token:.1f} us/token, {us_call:.2f} us/layer-token, "
          f"{bytes_call / us_call / 1e3:.0f} GB/s per layer call (lens ok {lens_ok}, status ok {status_ok})",
          file=sys.stderr, flush=True)
    del graphs, crop_graph

    # per-kernel durations, live: the same calls replayed eagerly with phase events
    ga.kv_crop(kvs, base_lens)
    nsteps_ev = min(args.steps, NSTEP, 26)
    pes, cfgs = [], []
    for s in range(nsteps_ev):
        for l in range(NL):
            pe = ga.PhaseEvents()
            c = ga.config(hidden=H, dtype=dtype, dispatch=args.dispatch, kv_split=args.kv_split)
            c.phase_events = pe.ptr
            pes.append(pe)
            cfgs.append(c)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)     # the GPU spins while the calls are enqueued: no enqueue gaps
    for i, c in enumerate(cfgs):
        s, l = divmod(i, NL)
        ga.layer_decode(c, weights[l], kvs[l], xs[s, l], outs[l], ws, host_lens=[P0 + s])
    torch.cuda.synchronize()
    ga.kv_crop(kvs, base_lens)
    durs = np.array([pe.elapsed_ms() for pe in pes]) * 1000.0     # [calls][3] us
    mean_us = dict(zip(PHASES, durs.mean(axis=0).tolist()))
    pb = [phase_bytes(H, 16, 8, 128, [P0 + s], 1) for s in range(nsteps_ev)]
    bphase = {k: float(np.mean([b[k] for b in pb])) for k in PHASES}
    print("[bench] bs1 phases (us): " + ", ".join(f"{k} {mean_us[k]:.2f}" for k in PHASES),
          file=sys.stderr, flush=True)

    verify = None if args.no_verify else verify_leg(ga, si, np, torch, dev, to_dev, stream, cfg, weights, kvs,
                                                    base_lens, H, NL, dtype, sid, P0)

    result = {
        "metric": "attn-block us/token (28 layers, bs1) + batched tok/s; % HBM roofline",
        "value": round(us_token, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(us_token / PAGES_US_PER_TOKEN, 5),
        "dtype": "f16 (fp32 arithmetic)",
        "data": "synthetic: seeded N(0,1) activations and cache, N(0,0.02) weights, norm gains 1+N(0,0.02)",
        "config": {"workload": "28-layer decoder attention, bs1, fp16, hidden 1024, 16q/8kv heads, head_dim 128, "
                               "KV 795->925 over 130 steps",
                   "layers": NL, "batch": 1, "hidden": H, "prefill": P0, "decode_steps": NSTEP,
                   "us_per_layer_token": round(us_call, 3),
                   "layer_call_gbs": round(bytes_call / us_call / 1e3, 1),
                   "layer_call_bytes": round(bytes_call),
                   "dispatch": args.dispatch, "kv_split": args.kv_split},
        "roofline": roofline(mean_us, bphase, measured_traffic("bs1")),
    }

    if verify is not None:
        result["verify"] = verify
    if not args.no_batched:
        result["batched"] = batched_leg(args, ga, si, np, torch, dev, to_dev, stream)
        if not args.no_wide:
            result["batched_h2048"] = wide_batched_leg(args, ga, si, np, torch, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


def batched_leg(args, ga, si, np, torch, dev, to_dev, stream):
    wl = si.WORKLOADS["ragged_batch64_h1024"]
    H, NL, B, dtype, sid = wl["hidden"], wl["layers"], wl["batch"], wl["dtype"], wl["stream"]
    lens = si.kv_lengths(sid, B, *wl["kv_len"])
    cfg = ga.config(hidden=H, dtype=dtype, dispatch=args.dispatch, kv_split=args.kv_split)
    t0 = time.time()
    weights, kvs = [], []
    for l in range(NL):
        wb = si.layer_weights(sid, l, H, dtype)
        weights.append(ga.Weights(*(to_dev(wb[n], dtype) for n in
                                    ("input_norm_w", "w_qkv", "q_norm_w", "k_norm_w", "w_o"))))
        kv = ga.KVLayer.empty(B, 8, CAP_B64, dtype=torch.bfloat16, device=dev)
        rows = si.kv_rows_many(sid, l, list(range(B)), lens.tolist(), dtype)
        for s, (kb, vb) in enumerate(rows):
            kv.k[s, :, : lens[s]] = to_dev(kb, dtype)
            kv.v[s, :, : lens[s]] = to_dev(vb, dtype)
        kv.lens.copy_(torch.from_numpy(lens))
        kvs.append(kv)
    xs = torch.stack([to_dev(si.activations(sid, l, 0, B, H, dtype), dtype) for l in range(NL)])
    outs = torch.empty((NL, B, H), dtype=torch.float32, device=dev)
    ws = ga.alloc_workspace(cfg, B, CAP_B64, device=dev)
    base = torch.from_numpy(lens.astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    print(f"[bench] batch-64 inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    hl = lens.tolist()
    if args.profile_batched:
        for _ in range(args.profile_batched):
            for l in range(NL):
                ga.layer_decode(cfg, weights[l], kvs[l], xs[l], outs[l], ws, host_lens=hl)
            ga.kv_crop(kvs, base)
        torch.cuda.synchronize()
        return None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(NL):
            ga.layer_decode(cfg, weights[l], kvs[l], xs[l], outs[l], ws, host_lens=hl)
        ga.kv_crop(kvs, base)
    ga.kv_crop(kvs, base)
    for _ in range(max(2, args.warmup // 4)):
        g.replay()
    torch.cuda.synchronize()
    n = max(10, args.steps // 4)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(n):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / n
    tok_s = B / (ms_step * 1e-3)
    bytes_step = NL * layer_bytes(H, 16, 8, 128, lens.tolist(), B)
    ok = all(int(kv.status.item()) == 0 for kv in kvs) and all(torch.equal(kv.lens, base) for kv in kvs)
    del g

    # per-kernel durations (eager, phase events): three steps of 28 layers
    pes, cfgs = [], []
    for _ in range(3 * NL):
        pe = ga.PhaseEvents()
        c = ga.config(hidden=H, dtype=dtype, dispatch=args.dispatch, kv_split=args.kv_split)
        c.phase_events = pe.ptr
        pes.append(pe)
        cfgs.append(c)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for i, c in enumerate(cfgs):
        l = i % NL
        ga.layer_decode(c, weights[l], kvs[l], xs[l], outs[l], ws, host_lens=hl)
        if l == NL - 1:
            ga.kv_crop(kvs, base)
    torch.cuda.synchronize()
    durs = np.array([pe.elapsed_ms() for pe in pes]) * 1000.0
    mean_us = dict(zip(PHASES, durs.mean(axis=0).tolist()))
    bphase = phase_bytes(H, 16, 8, 128, lens.tolist(), B)
    step_gbs = bytes_step / (ms_step * 1e-3) / 1e9
    print(f"[bench] batch-64: {ms_step * 1000:.1f} us/step, {tok_s:.0f} tok/s, {step_gbs:.0f} GB/s (ok {ok}); "
          "phases (us): " + ", ".join(f"{k} {mean_us[k]:.2f}" for k in PHASES), file=sys.stderr, flush=True)
    return {"workload": "28-layer ragged batched decode, 64 seqs, bf16, hidden 1024, KV U{200..1500}",
            "value": round(tok_s, 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 4), "steps": n,
            "step_gbs": round(step_gbs, 1), "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "roofline": roofline(mean_us, bphase, measured_traffic("b64"))}


def verify_leg(ga, si, np, torch, dev, to_dev, stream, cfg, weights, kvs, base_lens, H, NL, dtype, sid, P0):
    """k-token verify blocks at bs1 from the committed 795: 28 layer_verify calls captured in one
    graph, replayed with a crop back to 795 after each (the crop outside the timed events)."""
    out = {"workload": "28-layer verify block, bs1, fp16, hidden 1024, committed KV 795, k candidates",
           "unit": "us per 28-layer block"}
    ws_v = ga.alloc_workspace(cfg, 16, CAP_BS1, device=dev)
    for k in (4, 8, 16):
        xv = torch.stack([to_dev(si.activations(sid, l, 1000 + k, k, H, dtype).reshape(1, k, H), dtype)
                          for l in range(NL)])
        ov = torch.empty((NL, 1, k, H), dtype=torch.float32, device=dev)
        ga.kv_crop(kvs, base_lens)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(NL):
                ga.layer_verify(cfg, weights[l], kvs[l], xv[l], ov[l], ws_v, host_lens=[P0])
        crop = torch.cuda.CUDAGraph()
        with torch.cuda.graph(crop):
            ga.kv_crop(kvs, base_lens)
        for _ in range(5):
            g.replay()
            crop.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(40)]
        for e0, e1 in evs:
            e0.record(stream)
            g.replay()
            e1.record(stream)
            crop.replay()
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1000.0
        g.replay()
        torch.cuda.synchronize()
        ok = all(int(kv.lens.item()) == P0 + k and int(kv.status.item()) == 0 for kv in kvs)
        crop.replay()
        torch.cuda.synchronize()
        del g, crop
        out[f"k{k}"] = {"us_per_block": round(us, 2), "us_per_layer_block": round(us / NL, 3),
                        "us_per_candidate_token": round(us / k, 2), "ok": ok}
        print(f"[bench] verify bs1 k={k}: {us:.1f} us per 28-layer block, {us / NL:.2f} us per layer, "
              f"{us / k:.1f} us per candidate token (ok {ok})", file=sys.stderr, flush=True)
    return out


def wide_batched_leg(args, ga, si, np, torch, dev, stream):
    """Ragged batched decode at hidden 2048 (64 sequences, bf16, lengths uniform in [1024, 4096])
    and a k = 8 verify on 8 of them.  Weights and caches are drawn on the device from a seeded
    torch generator (the host generator would take minutes for 18 GB of caches); lengths and the
    verify choice come from the shared generator."""
    wl = si.WORKLOADS["ragged_batch64_h2048"]
    H, NL, B, dtype, sid = wl["hidden"], wl["layers"], wl["batch"], wl["dtype"], wl["stream"]
    k, nseq = wl["verify_k"][0], wl["verify_seqs"]
    lens = si.kv_lengths(sid, B, *wl["kv_len"])
    tdt = torch.bfloat16
    t0 = time.time()
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + sid)
    nqkv = (16 + 2 * 8) * 128

    def randn(shape, std=1.0, mean=0.0):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std + mean).to(tdt)

    weights, kvs = [], []
    for _ in range(NL):
        weights.append(ga.Weights(randn((H,), 0.02, 1.0), randn((nqkv, H), 0.02), randn((128,), 0.02, 1.0),
                                  randn((128,), 0.02, 1.0), randn((H, 16 * 128), 0.02)))
        kv = ga.KVLayer(randn((B, 8, CAP_W64, 128)), randn((B, 8, CAP_W64, 128)),
                        torch.from_numpy(lens.astype(np.int32)).to(dev), torch.zeros(1, dtype=torch.int32, device=dev))
        kvs.append(kv)
    xs = randn((NL, B, H))
    xv = randn((NL, nseq, k, H))
    outs = torch.empty((NL, B, H), dtype=torch.float32, device=dev)
    outv = torch.empty((NL, nseq, k, H), dtype=torch.float32, device=dev)
    cfg = ga.config(hidden=H, dtype=dtype, dispatch=args.dispatch, kv_split=args.kv_split)
    ws = ga.alloc_workspace(cfg, B, CAP_W64, device=dev)
    wsv = ga.alloc_workspace(cfg, nseq * k, CAP_W64, device=dev)
    base = torch.from_numpy(lens.astype(np.int32)).to(dev)
    chosen = si.verify_choice(sid, B, nseq)
    slots = torch.from_numpy(chosen).to(dev)
    hl, hlv = lens.tolist(), lens[chosen].tolist()
    torch.cuda.synchronize()
    print(f"[bench] batch-64 hidden 2048 inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def timed(calls, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        crop = torch.cuda.CUDAGraph()
        with torch.cuda.graph(crop):
            ga.kv_crop(kvs, base)
        for _ in range(3):
            g.replay()
            crop.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            e0.record(stream)
            g.replay()
            e1.record(stream)
            crop.replay()
        torch.cuda.synchronize()
        ok = all(int(kv.status.item()) == 0 for kv in kvs) and all(torch.equal(kv.lens, base) for kv in kvs)
        del g, crop
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])), ok

    def decode_calls():
        for l in range(NL):
            ga.layer_decode(cfg, weights[l], kvs[l], xs[l], outs[l], ws, host_lens=hl)

    def verify_calls():
        for l in range(NL):
            ga.layer_verify(cfg, weights[l], kvs[l], xv[l], outv[l], wsv, slots=slots, host_lens=hlv)

    ms_dec, ok_d = timed(decode_calls, max(10, args.steps // 8))
    ms_ver, ok_v = timed(verify_calls, max(10, args.steps // 8))
    bytes_step = NL * layer_bytes(H, 16, 8, 128, lens.tolist(), B)
    tok_s = B / (ms_dec * 1e-3)
    gbs = bytes_step / (ms_dec * 1e-3) / 1e9
    print(f"[bench] batch-64 hidden 2048: {ms_dec * 1000:.1f} us/step, {tok_s:.0f} tok/s, {gbs:.0f} GB/s (ok {ok_d}); "
          f"verify k={k} on {nseq} seqs: {ms_ver * 1000:.1f} us per 28-layer block (ok {ok_v})",
          file=sys.stderr, flush=True)
    del kvs, weights
    torch.cuda.empty_cache()
    return {"workload": "28-layer ragged batched decode, 64 seqs, bf16, hidden 2048, KV U{1024..4096}",
            "value": round(tok_s, 1), "unit": "tokens/s", "ms_per_step": round(ms_dec, 4),
            "step_gbs": round(gbs, 1), "step_hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "ok": ok_d,
            "verify": {"k": k, "sequences": nseq, "us_per_block": round(ms_ver * 1000, 1),
                       "us_per_layer_block": round(ms_ver * 1000 / NL, 2), "ok": ok_v}}


def cpu_baseline(budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the bs1 workload: the 28 layers of
    steps 0, 1, ... until the budget is spent; reported in microseconds per token."""
    import oracle
    from synth import inputs as si
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    wl = si.WORKLOADS["decode_bs1_28layers_kv795"]
    H, dtype, sid, P0, max_steps = wl["hidden"], wl["dtype"], wl["stream"], 795, 130
    ocfg = oracle.BlockConfig(hidden=H, dtype=dtype)
    layers = []
    for l in range(28):
        w = oracle.LayerWeights.from_bits(si.layer_weights(sid, l, H, dtype), dtype)
        kb, vb = si.kv_rows(sid, l, 0, P0, dtype)
        c = oracle.KVCache.empty(1, 8, CAP_BS1, 128, dtype)
        c.k[0, :, :P0], c.v[0, :, :P0], c.lens[0] = kb, vb, P0
        layers.append((w, c))
    calls, step = 0, 0
    t0 = time.perf_counter()
    while step < max_steps:
        for l in range(28):
            w, c = layers[l]
            oracle.decode(ocfg, w, c, si.activations(sid, l, step, 1, H, dtype))
            calls += 1
        step += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(dt / calls * 28 * 1e6, 1), "unit": "us/token", "cores": cores, "kind": "oracle",
            "sample": f"{step} decode steps x 28 layers of the bs1 workload (KV 795..{795 + step - 1}), "
                      f"fp64 NumPy oracle, {calls} layer calls in {dt:.1f}s"}


if __name__ == "__main__":
    main()
