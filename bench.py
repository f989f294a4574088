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
The timed region starts a round at step 0 and covers exactly ``--steps``
steps; ``config.workload`` names the committed lengths it covered.

Other legs (each can be skipped): ragged batched decode of 64 sequences in
bf16, committed lengths uniform in [200, 1500], with a 16-bit, an FP8 (E4M3)
and a paged 16-bit cache (``--no-batched``, ``--no-fp8``, ``--no-paged``); the
bs1 steps on paged caches (``--no-paged``; ``--page-size`` rows per page); the
bs1 verify block for k = 4, 8, 16 (``--no-verify``); the hidden-2048 batch-64
decode with a k = 8 verify on 8 sequences (``--no-wide``); the whole decoder's
greedy and speculative decoding (``--no-loop``).  Every leg reports its own roofline
(algorithmic bytes over the measured time, against 8 TB/s).

Per-kernel roofline: a second timed region replays the same calls eagerly with
HIP events that the library has the runtime stamp at the start and end of each
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
# logit gap below which two tokens count as tied in the batched speculative check: the one-token
# and block paths give the same logits to about 1e-3 (logits of about 3) after 28 layers whose
# outputs are rounded to 16 bits apart
NEAR_TIE = 5e-3
# HBM bytes per launch of each phase kernel from the FETCH_SIZE and WRITE_SIZE counters, each
# scaled by what that counter reads for a 1 GiB device copy (fetch x1.99992, write x1.000), and
# the digest of the kernel sources they were taken on: reported only while the sources match
TRAFFIC = {
    "sources_sha256": "4386e2f4ea80e25e43affc393d0c09996453fb1b49c96b35cd37c3b640228d91",
    "bs1": {"qkv_projection": 8587103, "attention": 4071800, "o_proj": 4885473},
    "b64": {"qkv_projection": 11059060, "attention": 230482124, "o_proj": 8712441},
    "b64_fp8": {"qkv_projection": 11059060, "attention": 120127730, "o_proj": 8712441},
    "b64_paged": {"qkv_projection": 11059060, "attention": 230736493, "o_proj": 8712441},
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
    return TRAFFIC.get(workload) if sources_digest() == TRAFFIC["sources_sha256"] else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=130)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-batched", action="store_true", help="skip the batch-64 workloads")
    p.add_argument("--no-verify", action="store_true", help="skip the bs1 verify blocks")
    p.add_argument("--no-wide", action="store_true", help="skip the hidden-2048 batch-64 workload")
    p.add_argument("--no-fp8", action="store_true", help="skip the batch-64 decode on an FP8 cache")
    p.add_argument("--no-paged", action="store_true", help="skip the batch-64 decode on a paged cache")
    p.add_argument("--page-size", type=int, default=16, help="rows per page of the paged batch-64 cache")
    p.add_argument("--no-loop", action="store_true",
                   help="skip greedy decoding and speculative rounds on the whole decoder with the model head")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    p.add_argument("--dispatch", type=int, default=0, help="0 auto, 1 one kernel per phase, 2 fused")
    p.add_argument("--kv-split", type=int, default=0, help="keys per split-KV chunk (0: automatic)")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="run only this many bs1 steps eagerly (for profilers) and exit")
    p.add_argument("--profile-batched", type=int, default=0,
                   help="run only this many batch-64 steps eagerly (for profilers) and exit")
    p.add_argument("--profile-verify", type=int, default=0,
                   help="run only this many bs1 verify blocks per k (and hidden-2048 verify blocks) eagerly and exit")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run three device-to-device copies of this many MiB (counter calibration)")
    return p.parse_args()


def phase_bytes(H, nq, nkv, d, committed, rows, e_in=2, e_out=4, e_kv=2):
    """Algorithmic HBM bytes of each phase of one layer call (workspace traffic not counted).

    qkv_projection: W_qkv, the three norm gains and x, read once.  attention: the committed K/V
    rows of every sequence read once and the appended K/V rows written (``e_kv`` bytes per cached
    element: 2, or 1 for an FP8 cache).  o_proj: W_o read once, out written."""
    qkv = ((nq + 2 * nkv) * d * H + H + 2 * d) * 2 + rows * H * e_in
    att = sum(committed) * 2 * nkv * d * e_kv + rows * 2 * nkv * d * e_kv
    oproj = H * nq * d * 2 + rows * H * e_out
    return {"qkv_projection": qkv, "attention": att, "o_proj": oproj}


def layer_bytes(H, nq, nkv, d, committed, rows, e_in=2, e_out=4, e_kv=2):
    return sum(phase_bytes(H, nq, nkv, d, committed, rows, e_in, e_out, e_kv).values())


def step_roofline(bytes_per_step, ms_per_step):
    """Whole-step rate: algorithmic bytes of every kernel of the step over the step's time."""
    gbs = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": round(bytes_per_step)}


# kernels one layer call launches (stream-ordered dispatch: projection, attention, o_proj)
KERNELS_PER_LAYER_CALL = 3


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
        if not args.no_fp8:
            batched_leg(args, ga, si, np, torch, dev, to_dev, stream, fp8=True)
        if not args.no_paged:
            batched_leg(args, ga, si, np, torch, dev, to_dev, stream, page=args.page_size)
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

    if args.profile_verify:
        verify_leg(ga, si, np, torch, dev, to_dev, stream, cfg, weights, kvs, base_lens, H, NL, dtype, sid, P0,
                   profile=args.profile_verify)
        if not args.no_wide:
            del weights, kvs
            torch.cuda.empty_cache()
            wide_batched_leg(args, ga, si, np, torch, dev, to_dev, stream)
        print(json.dumps({"profile_verify": args.profile_verify}))
        return

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
    if args.steps <= NSTEP:
        timed_kv = f"KV {P0}->{P0 + args.steps} ({args.steps} decode steps of a {NSTEP}-step round from {P0})"
    else:
        timed_kv = (f"KV {P0}->{P0 + NSTEP} ({args.steps} decode steps: {NSTEP}-step rounds from {P0}, "
                    f"a crop back to {P0} after each)")
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
    paged1 = None if args.no_paged else bs1_paged_leg(args, ga, si, np, torch, dev, to_dev, stream, cfg, weights, xs,
                                                      outs, ws, H, NL, dtype, sid, P0, NSTEP, args.page_size)

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
                               + timed_kv,
                   "layers": NL, "batch": 1, "hidden": H, "prefill": P0, "decode_steps": NSTEP,
                   "us_per_layer_token": round(us_call, 3),
                   "layer_call_gbs": round(bytes_call / us_call / 1e3, 1),
                   "layer_call_bytes": round(bytes_call),
                   "dispatch": args.dispatch, "kv_split": args.kv_split},
        "roofline": roofline(mean_us, bphase, measured_traffic("bs1")),
        "launches_per_token": round(NL * (1 if args.dispatch == 2 else KERNELS_PER_LAYER_CALL) + 1.0 / NSTEP, 3),
        "step_roofline": step_roofline(bytes_call * NL, ms_step),
    }

    if verify is not None:
        result["verify"] = verify
    if paged1 is not None:
        result["bs1_paged"] = paged1
    if not args.no_loop:
        result["verify_loop"] = loop_leg(args, ga, si, np, torch, dev, to_dev, stream)
    if not args.no_batched:
        result["batched"] = batched_leg(args, ga, si, np, torch, dev, to_dev, stream)
        if not args.no_fp8:
            result["batched_fp8"] = batched_leg(args, ga, si, np, torch, dev, to_dev, stream, fp8=True)
        if not args.no_paged:
            result["batched_paged"] = batched_leg(args, ga, si, np, torch, dev, to_dev, stream, page=args.page_size)
        if not args.no_wide:
            result["batched_h2048"] = wide_batched_leg(args, ga, si, np, torch, dev, to_dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bs1_paged_leg(args, ga, si, np, torch, dev, to_dev, stream, cfg, weights, xs, outs, ws, H, NL, dtype, sid, P0,
                  NSTEP, page):
    """The headline bs1 steps with every layer's cache a pool of `page`-row pages in shuffled
    order (the same prompt rows, inputs and timed steps)."""
    pps = CAP_BS1 // page
    table = torch.from_numpy(si.page_table(sid, 1, pps, pps)).to(dev)
    kvs = []
    for l in range(NL):
        kb, vb = si.kv_rows(sid, l, 0, P0, dtype)
        kv = ga.KVLayer.paged(pps, 8, page, table, dtype=torch.float16, device=dev)
        for bits, pool in ((kb, kv.k), (vb, kv.v)):
            full = torch.zeros((8, CAP_BS1, 128), dtype=torch.float16, device=dev)
            full[:, :P0] = to_dev(bits, dtype)
            pool[table[0].long()] = full.view(8, pps, page, 128).transpose(0, 1)
        kv.lens.fill_(P0)
        kvs.append(kv)
    base = torch.full((1,), P0, dtype=torch.int32, device=dev)
    graphs = []
    for s_ in range(NSTEP):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(NL):
                ga.layer_decode(cfg, weights[l], kvs[l], xs[s_, l], outs[l], ws, host_lens=[P0 + s_])
        graphs.append(g)
    crop = torch.cuda.CUDAGraph()
    with torch.cuda.graph(crop):
        ga.kv_crop(kvs, base)
    ga.kv_crop(kvs, base)
    torch.cuda.synchronize()

    def run(n):
        for i in range(n):
            graphs[i % NSTEP].replay()
            if i % NSTEP == NSTEP - 1:
                crop.replay()

    run(args.warmup)
    crop.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    run(args.steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    us_token = ev0.elapsed_time(ev1) / args.steps * 1000.0
    ok = all(int(kv.status.item()) == 0 for kv in kvs) and all(
        int(kv.lens.item()) == P0 + (args.steps % NSTEP) for kv in kvs)
    del graphs, crop, kvs
    torch.cuda.empty_cache()
    print(f"[bench] bs1 paged cache ({page}-row pages): {us_token:.1f} us/token (ok {ok})", file=sys.stderr, flush=True)
    return {"workload": f"the bs1 steps above on paged caches of {page}-row pages in shuffled order",
            "value": round(us_token, 3), "unit": "us/token", "page_size": page, "ok": ok}


def batched_leg(args, ga, si, np, torch, dev, to_dev, stream, fp8=False, page=0):
    """Ragged batched decode of 64 sequences (bf16, hidden 1024, lengths uniform in [200, 1500]):
    one step = 28 layer calls + the crop back to the committed lengths, graph-replayed.  With
    ``fp8`` the caches hold E4M3 codes of the same draws with per-kv-head scales; with ``page``
    each layer's cache is a pool of pages of that many rows, every sequence's pages in a shuffled
    order (a pool whose pages many requests have taken and returned)."""
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
        if fp8:
            ks, vs = si.kv_scales(sid, l)
            kv = ga.KVLayer.empty(B, 8, CAP_B64, dtype=torch.uint8, device=dev,
                                  k_scale=torch.from_numpy(ks).to(dev), v_scale=torch.from_numpy(vs).to(dev))
            rows = si.kv_rows_e4m3_many(sid, l, list(range(B)), lens.tolist(), ks, vs)
            for s_, (kc, vc) in enumerate(rows):
                kv.k[s_, :, : lens[s_]] = torch.from_numpy(kc).to(dev)
                kv.v[s_, :, : lens[s_]] = torch.from_numpy(vc).to(dev)
        elif page:
            pps = CAP_B64 // page
            table = torch.from_numpy(si.page_table(sid, B, pps, B * pps)).to(dev)
            kv = ga.KVLayer.paged(B * pps, 8, page, table, dtype=torch.bfloat16, device=dev)
            rows = si.kv_rows_many(sid, l, list(range(B)), lens.tolist(), dtype)
            for s_, (kb, vb) in enumerate(rows):
                for which, bits, pool in (("k", kb, kv.k), ("v", vb, kv.v)):
                    full = torch.zeros((8, CAP_B64, 128), dtype=torch.bfloat16, device=dev)
                    full[:, : lens[s_]] = to_dev(bits, dtype)
                    pool[table[s_].long()] = full.view(8, pps, page, 128).transpose(0, 1)
        else:
            kv = ga.KVLayer.empty(B, 8, CAP_B64, dtype=torch.bfloat16, device=dev)
            rows = si.kv_rows_many(sid, l, list(range(B)), lens.tolist(), dtype)
            for s_, (kb, vb) in enumerate(rows):
                kv.k[s_, :, : lens[s_]] = to_dev(kb, dtype)
                kv.v[s_, :, : lens[s_]] = to_dev(vb, dtype)
        kv.lens.copy_(torch.from_numpy(lens))
        kvs.append(kv)
    xs = torch.stack([to_dev(si.activations(sid, l, 0, B, H, dtype), dtype) for l in range(NL)])
    outs = torch.empty((NL, B, H), dtype=torch.float32, device=dev)
    ws = ga.alloc_workspace(cfg, B, CAP_B64, device=dev)
    base = torch.from_numpy(lens.astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    tag = "batch-64 fp8 cache" if fp8 else (f"batch-64 paged cache ({page}-row pages)" if page else "batch-64")
    print(f"[bench] {tag} inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
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
    e_kv = 1 if fp8 else 2
    bytes_step = NL * layer_bytes(H, 16, 8, 128, lens.tolist(), B, e_kv=e_kv)
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
    bphase = phase_bytes(H, 16, 8, 128, lens.tolist(), B, e_kv=e_kv)
    sr = step_roofline(bytes_step, ms_step)
    print(f"[bench] {tag}: {ms_step * 1000:.1f} us/step, {tok_s:.0f} tok/s, {sr['achieved']:.0f} GB/s (ok {ok}); "
          "phases (us): " + ", ".join(f"{k} {mean_us[k]:.2f}" for k in PHASES), file=sys.stderr, flush=True)
    del kvs, weights
    torch.cuda.empty_cache()
    cache = ("FP8 (E4M3) cache with per-kv-head scales" if fp8 else
             f"bf16 paged cache, {page}-row pages in shuffled order" if page else "bf16 cache")
    tkey = "b64_fp8" if fp8 else ("b64_paged" if page else "b64")
    return {"workload": "28-layer ragged batched decode, 64 seqs, bf16 weights, " + cache
                        + ", hidden 1024, KV U{200..1500}",
            "value": round(tok_s, 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 4), "steps": n,
            "step_roofline": sr, "ok": ok,
            "roofline": roofline(mean_us, bphase, measured_traffic(tkey))}


def verify_leg(ga, si, np, torch, dev, to_dev, stream, cfg, weights, kvs, base_lens, H, NL, dtype, sid, P0,
               profile=0):
    """k-token verify blocks at bs1 from the committed 795: 28 layer_verify calls captured in one
    graph, replayed with a crop back to 795 after each (the crop timed on its own events).  With
    ``profile``: that many blocks per k, eagerly, for profilers."""
    out = {"workload": "28-layer verify block, bs1, fp16, hidden 1024, committed KV 795, k candidates",
           "unit": "us per 28-layer block"}
    ws_v = ga.alloc_workspace(cfg, 16, CAP_BS1, device=dev)
    for k in (4, 8, 16):
        xv = torch.stack([to_dev(si.activations(sid, l, 1000 + k, k, H, dtype).reshape(1, k, H), dtype)
                          for l in range(NL)])
        ov = torch.empty((NL, 1, k, H), dtype=torch.float32, device=dev)
        ga.kv_crop(kvs, base_lens)
        torch.cuda.synchronize()
        if profile:
            for _ in range(profile):
                for l in range(NL):
                    ga.layer_verify(cfg, weights[l], kvs[l], xv[l], ov[l], ws_v, host_lens=[P0])
                ga.kv_crop(kvs, base_lens)
            torch.cuda.synchronize()
            continue
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
        cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(40)]
        for (e0, e1), (c0, c1) in zip(evs, cevs):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            c0.record(stream)
            crop.replay()
            c1.record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1000.0
        crop_us = float(np.mean([c0.elapsed_time(c1) for c0, c1 in cevs])) * 1000.0
        g.replay()
        torch.cuda.synchronize()
        ok = all(int(kv.lens.item()) == P0 + k and int(kv.status.item()) == 0 for kv in kvs)
        crop.replay()
        torch.cuda.synchronize()
        del g, crop
        b_layer = layer_bytes(H, 16, 8, 128, [P0], k)
        gbs = b_layer / (us / NL * 1e-6) / 1e9
        out[f"k{k}"] = {"us_per_block": round(us, 2), "us_per_layer_block": round(us / NL, 3),
                        "us_per_candidate_token": round(us / k, 2), "ok": ok,
                        "crop_us": round(crop_us, 2),   # the 28 layers' crop back to 795, one dispatch
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_layer_block": b_layer}}
        print(f"[bench] verify bs1 k={k}: {us:.1f} us per 28-layer block, {us / NL:.2f} us per layer, "
              f"{us / k:.1f} us per candidate token (ok {ok})", file=sys.stderr, flush=True)
    return out


def wide_batched_leg(args, ga, si, np, torch, dev, to_dev, stream):
    """Ragged batched decode at hidden 2048 (64 sequences, bf16, lengths uniform in [1024, 4096])
    and a k = 8 verify on 8 of them.  Every input comes from the shared seeded generator: the
    weights and activations of each layer, and the caches of layer 0, which the other 27 layers
    receive as device copies (drawing 18 GB of cache rows on the host would take minutes; the
    values do not change the work)."""
    from concurrent.futures import ThreadPoolExecutor
    wl = si.WORKLOADS["ragged_batch64_h2048"]
    H, NL, B, dtype, sid = wl["hidden"], wl["layers"], wl["batch"], wl["dtype"], wl["stream"]
    k, nseq = wl["verify_k"][0], wl["verify_seqs"]
    lens = si.kv_lengths(sid, B, *wl["kv_len"])
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        wbits = list(ex.map(lambda l: si.layer_weights(sid, l, H, dtype), range(NL)))
    weights = [ga.Weights(*(to_dev(wb[n], dtype) for n in ("input_norm_w", "w_qkv", "q_norm_w", "k_norm_w", "w_o")))
               for wb in wbits]
    del wbits
    kv0 = ga.KVLayer.empty(B, 8, CAP_W64, dtype=torch.bfloat16, device=dev)
    for s_, (kb, vb) in enumerate(si.kv_rows_many(sid, 0, list(range(B)), lens.tolist(), dtype)):
        kv0.k[s_, :, : lens[s_]] = to_dev(kb, dtype)
        kv0.v[s_, :, : lens[s_]] = to_dev(vb, dtype)
    kvs = [kv0]
    for _ in range(1, NL):
        kvs.append(ga.KVLayer(kv0.k.clone(), kv0.v.clone(), torch.zeros(B, dtype=torch.int32, device=dev),
                              torch.zeros(1, dtype=torch.int32, device=dev)))
    for kv in kvs:
        kv.lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    xs = torch.stack([to_dev(si.activations(sid, l, 0, B, H, dtype), dtype) for l in range(NL)])
    xv = torch.stack([to_dev(si.activations(sid, l, 1, nseq * k, H, dtype).reshape(nseq, k, H), dtype)
                      for l in range(NL)])
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

    if args.profile_verify:
        for _ in range(args.profile_verify):
            verify_calls()
            ga.kv_crop(kvs, base)
        torch.cuda.synchronize()
        return None
    ms_dec, ok_d = timed(decode_calls, max(10, args.steps // 8))
    ms_ver, ok_v = timed(verify_calls, max(10, args.steps // 8))
    bytes_step = NL * layer_bytes(H, 16, 8, 128, lens.tolist(), B)
    bytes_ver = NL * layer_bytes(H, 16, 8, 128, lens[chosen].tolist(), nseq * k)
    tok_s = B / (ms_dec * 1e-3)
    gbs = bytes_step / (ms_dec * 1e-3) / 1e9
    print(f"[bench] batch-64 hidden 2048: {ms_dec * 1000:.1f} us/step, {tok_s:.0f} tok/s, {gbs:.0f} GB/s (ok {ok_d}); "
          f"verify k={k} on {nseq} seqs: {ms_ver * 1000:.1f} us per 28-layer block (ok {ok_v})",
          file=sys.stderr, flush=True)
    del kvs, weights
    torch.cuda.empty_cache()
    return {"workload": "28-layer ragged batched decode, 64 seqs, bf16, hidden 2048, KV U{1024..4096}",
            "value": round(tok_s, 1), "unit": "tokens/s", "ms_per_step": round(ms_dec, 4),
            "step_roofline": step_roofline(bytes_step, ms_dec), "ok": ok_d,
            "verify": {"k": k, "sequences": nseq, "us_per_block": round(ms_ver * 1000, 1),
                       "us_per_layer_block": round(ms_ver * 1000 / NL, 2), "ok": ok_v,
                       "roofline": step_roofline(bytes_ver, ms_ver)}}


def loop_leg(args, ga, si, np, torch, dev, to_dev, stream):
    """Greedy decoding and speculative rounds with an oracle draft on the whole decoder: 28 layers
    of attention + MLP (hidden 1024, intermediate 3072), the token embedding and the final norm +
    lm_head argmax over 151,936 ids, bs1 fp16, a 795-token prompt ("Can CTC make Qwen3-ASR
    faster?", section 11 Phase A steps 2-4: verify_block, the one-token shift, an oracle draft,
    block sizes).  Greedy: one captured graph per token (embedding, 28 layer decodes, argmax fed
    back as the next input).  Speculative: one graph per round of k (embedding of the block, 28
    layer verifies, argmax of every row, acceptance, crop); the draft is the greedy transcript, so
    every round commits k tokens.  Reported in microseconds per committed token."""
    from concurrent.futures import ThreadPoolExecutor
    H, I, V, NL, P0, dtype, sid = 1024, 3072, 151936, 28, 795, si.F16, 6
    T = 64                                     # tokens per timed pass
    cap = P0 + T + 16
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        wa = list(ex.map(lambda l: si.layer_weights(sid, l, H, dtype), range(NL)))
        wm = list(ex.map(lambda l: si.mlp_weights(sid, l, H, I, dtype), range(NL)))
        kvb = list(ex.map(lambda l: si.kv_rows(sid, l, 0, P0, dtype), range(NL)))
    hb = si.head_weights(sid, H, V, dtype)
    aw = [ga.Weights(*(to_dev(w[n], dtype) for n in ("input_norm_w", "w_qkv", "q_norm_w", "k_norm_w", "w_o"))) for w in wa]
    mw = [ga.MlpWeights(*(to_dev(w[n], dtype) for n in ("post_norm_w", "w_gate", "w_up", "w_down"))) for w in wm]
    table, gfin, wlm = to_dev(hb["embed"], dtype), to_dev(hb["final_norm_w"], dtype), to_dev(hb["w_lm"], dtype)
    del wa, wm, hb
    kvs = []
    for kb, vb in kvb:
        kv = ga.KVLayer.empty(1, 8, cap, dtype=torch.float16, device=dev)
        kv.k[0, :, :P0], kv.v[0, :, :P0] = to_dev(kb, dtype), to_dev(vb, dtype)
        kv.lens.fill_(P0)
        kvs.append(kv)
    kvb_first = kvb
    base = torch.full((1,), P0, dtype=torch.int32, device=dev)
    acfg = ga.config(hidden=H, dtype=dtype)
    mcfg, mlast = ga.mlp_config(hidden=H, intermediate=I, dtype=dtype, out_dtype=dtype), ga.mlp_config(hidden=H, intermediate=I, dtype=dtype)
    hcfg = ga.head_config(hidden=H, vocab=V, dtype=dtype)
    KMAX = 16
    ws = ga.decoder_layer_workspace(acfg, mcfg, KMAX, cap, device=dev)
    hws = ga.lm_head_workspace(hcfg, KMAX, device=dev)
    xa = torch.empty((KMAX, H), dtype=torch.float16, device=dev)
    xb = torch.empty((KMAX, H), dtype=torch.float16, device=dev)
    hf = torch.empty((KMAX, H), dtype=torch.float32, device=dev)
    print(f"[bench] loop model ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def forward(ids, n, L, out_ids):
        """ids [n] -> out_ids [n]: the block through the 28 layers and the head (L = committed length)."""
        ga.embed(table, ids, xa[:n])
        x = xa
        for l in range(NL):
            last = l == NL - 1
            o = hf if last else (xb if x is xa else xa)
            if n == 1:
                ga.decoder_layer_decode(acfg, aw[l], mlast if last else mcfg, mw[l], kvs[l], x[:1], o[:1], ws,
                                        host_lens=[L])
            else:
                ga.decoder_layer_verify(acfg, aw[l], mlast if last else mcfg, mw[l], kvs[l], x[:n].view(1, n, H),
                                        o[:n].view(1, n, H), ws, host_lens=[L])
            x = o
        ga.lm_head_argmax(hcfg, gfin, wlm, hf[:n], out_ids, hws)

    # the greedy transcript (untimed), then the timed greedy graphs: the argmax feeds the next step
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    trans = []
    for s_ in range(T):
        forward(tok, 1, P0 + s_, tok)
        trans.append(tok.clone())
    trans = torch.cat(trans)
    ga.kv_crop(kvs, base)
    tok.zero_()
    torch.cuda.synchronize()
    graphs = []
    for s_ in range(T):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            forward(tok, 1, P0 + s_, tok)
        graphs.append(g)
    ga.kv_crop(kvs, base)
    torch.cuda.synchronize()

    def time_graphs(gs, reps=3):
        best = None
        for _ in range(reps):
            tok.zero_()
            ga.kv_crop(kvs, base)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for g in gs:
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    ms_greedy = time_graphs(graphs)
    # the graphs reproduce the transcript
    tok.zero_()
    ga.kv_crop(kvs, base)
    replay = []
    for g in graphs:
        g.replay()
        replay.append(tok.clone())
    greedy_ok = bool(torch.equal(torch.cat(replay), trans))
    del graphs
    out = {"workload": "greedy decoding and speculative rounds, 28 decoder layers (attention + MLP, hidden 1024, "
                       "intermediate 3072) + embedding + final norm + lm_head argmax (151,936 ids), bs1, fp16, "
                       f"prompt {P0}, {T} tokens per pass, oracle draft (the greedy transcript)",
           "unit": "us per committed token",
           "greedy": {"us_per_token": round(ms_greedy * 1000 / T, 2), "ok": greedy_ok}}
    print(f"[bench] loop greedy: {ms_greedy * 1000 / T:.1f} us/token (ok {greedy_ok})", file=sys.stderr, flush=True)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    new_lens = torch.empty(1, dtype=torch.int32, device=dev)
    for k in (4, 8, 16):
        R = T // k
        blocks = torch.stack([torch.cat([start if j == 0 else trans[j * k - 1:j * k], trans[j * k:j * k + k - 1]])
                              for j in range(R)]).contiguous()
        drafts = torch.stack([trans[j * k:(j + 1) * k] for j in range(R)]).contiguous()
        tgt = torch.empty((R, k), dtype=torch.int32, device=dev)
        accs = torch.empty(R, dtype=torch.int32, device=dev)
        gs = []
        for j in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                forward(blocks[j], k, P0 + j * k, tgt[j])
                ga.accept_greedy(drafts[j:j + 1], tgt[j:j + 1], kvs[0].lens, accs[j:j + 1], nxt, new_lens)
                ga.kv_crop(kvs, new_lens)
            gs.append(g)
        ga.kv_crop(kvs, base)
        torch.cuda.synchronize()
        ms = time_graphs(gs)
        ok = bool(torch.all(accs == k).item()) and int(kvs[0].lens.item()) == P0 + R * k
        del gs
        out[f"k{k}"] = {"us_per_committed_token": round(ms * 1000 / (R * k), 2), "us_per_round": round(ms * 1000 / R, 1),
                        "rounds": R, "accepted_per_round": k, "ok": ok,
                        "speedup_vs_greedy": round(ms_greedy / ms, 3)}
        print(f"[bench] loop speculative k={k}: {ms * 1000 / (R * k):.1f} us per committed token, "
              f"{ms * 1000 / R:.1f} us per round (ok {ok})", file=sys.stderr, flush=True)
    del kvs
    torch.cuda.empty_cache()
    out["batched"] = spec_batch_leg(ga, si, np, torch, dev, to_dev, kvb_first, aw, mw, table, gfin, wlm,
                                    H, I, V, NL, dtype, sid)
    del aw, mw, table, wlm
    torch.cuda.empty_cache()
    return out


def spec_batch_leg(ga, si, np, torch, dev, to_dev, prompt_rows, aw, mw, table, gfin, wlm, H, I, V, NL, dtype, sid):
    """Batched speculative decoding with per-sequence block lengths on the whole decoder ("Can CTC
    make Qwen3-ASR faster?", section 07 and section 08 "Verifier, version 0"; section 12's fixed
    block sizes against entropy-adaptive ones).  16 sequences with prompts of 150 to 795 positions
    (the first rows of each layer's bs1 prompt); drafts are each sequence's greedy transcript with
    seeded substitutions, insertions and deletions at a rate of 1 in 12, and uncertainties that flag
    them.  Every round: the blocks of the active sequences packed into one mixed batch (embedding,
    28 mixed decoder layers, argmax of every row, acceptance per sequence, crop), then the host picks
    each sequence's next block length and recycles its draft.  Device time per round is taken
    between events while the host has already enqueued the round (the GPU spins meanwhile), so it
    holds no host gaps; committed tokens per second of that time, against greedy batched decoding
    timed the same way."""
    B, T, P_hi = 16, 48, 795
    prompts = [150 + (P_hi - 150) * s // (B - 1) for s in range(B)]
    cap = P_hi + T + 32
    KMAX = 16
    kvs = []
    for l in range(NL):
        kv = ga.KVLayer.empty(B, 8, cap, dtype=torch.float16, device=dev)
        kb, vb = prompt_rows[l]
        kd, vd = to_dev(kb, dtype), to_dev(vb, dtype)
        for s_, P in enumerate(prompts):
            kv.k[s_, :, :P], kv.v[s_, :, :P] = kd[:, :P], vd[:, :P]
        kv.lens.copy_(torch.tensor(prompts, dtype=torch.int32))
        kvs.append(kv)
    base = torch.tensor(prompts, dtype=torch.int32, device=dev)
    acfg = ga.config(hidden=H, dtype=dtype)
    mcfg = ga.mlp_config(hidden=H, intermediate=I, dtype=dtype, out_dtype=dtype)
    mlast = ga.mlp_config(hidden=H, intermediate=I, dtype=dtype)
    hcfg = ga.head_config(hidden=H, vocab=V, dtype=dtype)
    ws = ga.decoder_layer_workspace(acfg, mcfg, B * KMAX, cap, device=dev)
    hws = ga.lm_head_workspace(hcfg, B * KMAX, device=dev)
    xa = torch.empty((B * KMAX, H), dtype=torch.float16, device=dev)
    xb = torch.empty((B * KMAX, H), dtype=torch.float16, device=dev)
    hf = torch.empty((B * KMAX, H), dtype=torch.float32, device=dev)
    tgt = torch.empty(B * KMAX, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    new_lens = torch.empty(B, dtype=torch.int32, device=dev)
    first = [(7919 * (s_ + 1)) % V for s_ in range(B)]

    def run_block(ids, sizes, slots):
        rows = sum(sizes)
        ga.embed(table, ids, xa[:rows])
        x = xa
        for l in range(NL):
            last = l == NL - 1
            o = hf if last else (xb if x is xa else xa)
            ga.decoder_layer_mixed(acfg, aw[l], mlast if last else mcfg, mw[l], kvs[l], x[:rows], sizes, o[:rows], ws,
                                   slots=slots)
            x = o
        ga.lm_head_argmax(hcfg, gfin, wlm, hf[:rows], tgt[:rows], hws)

    def timed(enqueue):
        """Device time of the enqueued work, free of host gaps."""
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(10_000_000)
        e0.record()
        enqueue()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # greedy transcripts (untimed), then greedy batched decoding timed step by step
    ga.kv_crop(kvs, base)
    cur = torch.tensor(first, dtype=torch.int32, device=dev)
    allslots = torch.arange(B, dtype=torch.int32, device=dev)
    trans, gaps = [], []
    w32, g32 = wlm.float(), gfin.float()
    for _ in range(T + 24):
        run_block(cur, [1] * B, allslots)
        cur = tgt[:B].clone()
        trans.append(cur.cpu().tolist())
        # the top-two logit gap of every greedy token (fp32 logits, for the check below)
        y = hf[:B] * torch.rsqrt((hf[:B] * hf[:B]).mean(dim=1, keepdim=True) + 1e-6) * g32
        top = torch.topk(y @ w32.t(), 2, dim=1).values
        gaps.append((top[:, 0] - top[:, 1]).cpu().tolist())
    del w32
    trans = [[trans[t][s_] for t in range(T + 24)] for s_ in range(B)]
    ga.kv_crop(kvs, base)
    cur = torch.tensor(first, dtype=torch.int32, device=dev)
    ms_greedy = 0.0
    for t in range(T):
        ms_greedy += timed(lambda: run_block(cur, [1] * B, allslots))
        cur = tgt[:B].clone()
    greedy_ok = all(x == trans[s_][T - 1] for s_, x in enumerate(cur.cpu().tolist()))
    tok_greedy = B * T / (ms_greedy * 1e-3)
    res = {"workload": f"batched speculative decoding, {B} sequences, prompts {prompts[0]}..{prompts[-1]}, "
                       f"{T} tokens each, 28 decoder layers + head (151,936 ids), fp16; drafts: greedy transcripts "
                       "with seeded substitutions, insertions and deletions (1 in 12) and uncertainties flagging them",
           "unit": "committed tokens/s (device time)",
           "greedy": {"tokens_per_s": round(tok_greedy, 1), "ms": round(ms_greedy, 3), "ok": greedy_ok}}
    print(f"[bench] batched greedy: {tok_greedy:.0f} tok/s ({ms_greedy:.2f} ms for {B}x{T}; ok {greedy_ok})",
          file=sys.stderr, flush=True)
    drafts = [si.draft_with_edits(sid, s_, trans[s_], 1 / 12, V) for s_ in range(B)]
    variants = {"fixed_k8": (8, 8, 0, 1e30), "fixed_k8_recycle2": (8, 8, 2, 1e30), "adaptive_2_16_recycle2": (2, 16, 2, 1.0)}
    for name, (kmin, kmax, window, tau) in variants.items():
        ga.kv_crop(kvs, base)
        pos, last = [0] * B, list(first)
        got = [[] for _ in range(B)]
        done = [False] * B
        ms, rounds, rows_total, acc_total = 0.0, 0, 0, 0
        while not all(done):
            act = [s_ for s_ in range(B) if not done[s_]]
            kk = [ga.next_block_len(drafts[s_][1][pos[s_]:], tau, kmin, kmax) for s_ in act]
            dr = [(drafts[s_][0][pos[s_]:] + [-1] * k)[:k] for s_, k in zip(act, kk)]
            ids = torch.tensor([t for s_, d, k in zip(act, dr, kk) for t in [last[s_]] + d[:k - 1]],
                               dtype=torch.int32, device=dev)
            dflat = torch.tensor([t for d in dr for t in d], dtype=torch.int32, device=dev)
            slots = torch.tensor(act, dtype=torch.int32, device=dev)

            def enqueue():
                run_block(ids, kk, slots)
                ga.accept_greedy_mixed(dflat, tgt[:sum(kk)], kk, kvs[0].lens, acc[:len(act)], nxt[:len(act)],
                                       new_lens, slots=slots)
                ga.kv_crop(kvs, new_lens)
            ms += timed(enqueue)
            A, N = acc[:len(act)].cpu().tolist(), nxt[:len(act)].cpu().tolist()
            for i, s_ in enumerate(act):
                k, a = kk[i], A[i]
                got[s_] += dr[i][:a] + ([] if a == k else [N[i]])
                pos[s_] = ga.recycle_draft(drafts[s_][0], pos[s_], k, a, None if a == k else N[i], window)
                last[s_] = got[s_][-1]
                done[s_] = len(got[s_]) >= T
            rounds += 1
            rows_total += sum(kk)
            acc_total += sum(A)
        # greedy exactness: each transcript equals the greedy one, or first leaves it at a token
        # whose two best logits lie closer than the rounding of the two computations can tell
        # apart (the block path and the one-token path round each layer's 16-bit output apart)
        exact, ties = 0, []
        for s_ in range(B):
            dv = next((t for t in range(T) if got[s_][t] != trans[s_][t]), None)
            if dv is None:
                exact += 1
            else:
                ties.append({"seq": s_, "pos": dv, "greedy_top2_gap": round(gaps[dv][s_], 6)})
        ok = all(t["greedy_top2_gap"] < NEAR_TIE for t in ties)
        committed = sum(len(g) for g in got)
        tps = committed / (ms * 1e-3)
        res[name] = {"tokens_per_s": round(tps, 1), "ms": round(ms, 3), "rounds": rounds,
                     "committed": committed, "rows_verified": rows_total,
                     "committed_per_row": round(committed / rows_total, 3), "ok": ok,
                     "exact_sequences": exact, "near_tie_divergences": ties,
                     "speedup_vs_greedy": round(tps / tok_greedy, 3)}
        print(f"[bench] batched speculative {name}: {tps:.0f} tok/s, {rounds} rounds, "
              f"{committed / rows_total:.2f} committed per verified row, {exact}/{B} transcripts exact, "
              f"other divergences at near ties {[t['greedy_top2_gap'] for t in ties]} (ok {ok})",
              file=sys.stderr, flush=True)
    del kvs
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s):
    """The fp64 oracle, as it stands, on bounded samples: the bs1 decode workload with all host
    threads (the 28 layers of steps 0, 1, ... until the budget is spent; us per token), then with
    one thread the single-layer KV-64 call and the 28-layer verify blocks (k = 4, 8, 16) from 795."""
    import oracle
    from synth import inputs as si
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
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
    base = [c.copy() for _, c in layers]
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
    out = {"value": round(dt / calls * 28 * 1e6, 1), "unit": "us/token", "cores": cores, "kind": "oracle",
           "cpu": cpu_model(),
           "sample": f"{step} decode steps x 28 layers of the bs1 workload (KV 795..{795 + step - 1}), "
                     f"fp64 NumPy oracle on {cores} threads, {calls} layer calls in {dt:.1f}s"}
    with threadpool_limits(limits=1):
        w1 = si.WORKLOADS["decode_bs1_1layer_kv64"]
        s1 = w1["stream"]
        o1 = oracle.BlockConfig(hidden=w1["hidden"], dtype=w1["dtype"])
        wt = oracle.LayerWeights.from_bits(si.layer_weights(s1, 0, w1["hidden"], w1["dtype"]), w1["dtype"])
        kb, vb = si.kv_rows(s1, 0, 0, 64, w1["dtype"])
        reps, t1 = 0, time.perf_counter()
        while reps < 20 or time.perf_counter() - t1 < 1.0:
            c = oracle.KVCache.empty(1, 8, 128, 128, w1["dtype"])
            c.k[0, :, :64], c.v[0, :, :64], c.lens[0] = kb, vb, 64
            oracle.decode(o1, wt, c, si.activations(s1, 0, 0, 1, w1["hidden"], w1["dtype"]))
            reps += 1
        out["one_thread_single_layer_kv64_us_per_call"] = round((time.perf_counter() - t1) / reps * 1e6, 1)
        w3 = si.WORKLOADS["verify_bs1_28layers_kv795"]
        ver = {}
        for k in w3["verify_k"]:
            caches = [c.copy() for c in base]
            t3 = time.perf_counter()
            for l in range(28):
                oracle.verify(ocfg, layers[l][0], caches[l], si.activations(sid, l, 1000 + k, k, H, dtype)[None])
            ver[f"k{k}"] = round((time.perf_counter() - t3) * 1e6, 1)
        out["one_thread_verify_28_layers_us_per_block"] = ver
    return out


if __name__ == "__main__":
    main()
