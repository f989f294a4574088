"""HIP graph capture and replay of layer calls.

A step of several layer calls is captured once and replayed several times.
Between replays the program does its own eager work on the same buffers: new
inputs copied into the captured ones, a crop of every layer back to the
captured start, eager layer calls on the same workspace, host synchronisation.
Every replay must leave the outputs, cache bits and lengths that eager calls
on the same inputs leave, and the first replay is also checked against the
oracle.
"""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import TOL, SeededLayer, device_cache, fill_cache, oracle_cache, rel_err, tdt, to_bits, to_dev

pytestmark = pytest.mark.gpu

NL, H, REPLAYS = 2, 1024, 4
# name: dtype, committed lengths, rows per sequence (1 decode, k verify), capacity, dispatch
CASES = {
    "bs1_f16": (si.F16, [300], 1, 320, ga.DISPATCH_MULTI),
    "bs1_f16_one_dispatch": (si.F16, [300], 1, 320, ga.DISPATCH_FUSED),
    "ragged12_bf16": (si.BF16, [37, 250, 5, 120, 64, 300, 17, 200, 90, 1, 150, 280], 1, 320, ga.DISPATCH_MULTI),
    "verify3x4_f16": (si.F16, [100, 33, 260], 4, 320, ga.DISPATCH_MULTI),
}


def _inputs(step, B, n, dtype):
    """[NL][B][n][H] bits of one step's layer inputs."""
    return np.stack([si.activations(9, l, step, B * n, H, dtype).reshape(B, n, H) for l in range(NL)])


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_equal_eager_calls(case):
    dtype, lens, n, cap, dispatch = CASES[case]
    B = len(lens)
    layers = [SeededLayer(9, l, H, dtype) for l in range(NL)]
    caches = [fill_cache(9, l, lens, cap, dtype) for l in range(NL)]
    kvs = [device_cache(kb, vb, lens, dtype) for kb, vb in caches]
    base = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    cfg = ga.config(dtype=dtype, dispatch=dispatch)
    ws = ga.alloc_workspace(cfg, B * n, cap)
    x = torch.empty((NL, B, n, H), dtype=tdt(dtype), device="cuda")
    out = torch.empty((NL, B, n, H), dtype=torch.float32, device="cuda")

    def step_calls():
        for l in range(NL):
            if n == 1:
                ga.layer_decode(cfg, layers[l].dev, kvs[l], x[l, :, 0], out[l, :, 0], ws, host_lens=lens)
            else:
                ga.layer_verify(cfg, layers[l].dev, kvs[l], x[l], out[l], ws, host_lens=lens)

    def state():
        torch.cuda.synchronize()
        return (out.cpu().numpy().copy(), [to_bits(kv.k) for kv in kvs], [to_bits(kv.v) for kv in kvs],
                [kv.lens.cpu().numpy() for kv in kvs], [int(kv.status.item()) for kv in kvs])

    # eager results of each replay's inputs, each from the captured start
    eager = []
    for r in range(REPLAYS):
        ga.kv_crop(kvs, base)
        x.copy_(to_dev(_inputs(r, B, n, dtype), dtype))
        step_calls()
        eager.append(state())

    ga.kv_crop(kvs, base)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_calls()
    for r in range(REPLAYS):
        ga.kv_crop(kvs, base)
        if r % 2 == 1:
            # eager calls on the same workspace between replays, then back to the start
            x.copy_(to_dev(_inputs(100 + r, B, n, dtype), dtype))
            step_calls()
            torch.cuda.synchronize()
            ga.kv_crop(kvs, base)
        x.copy_(to_dev(_inputs(r, B, n, dtype), dtype))
        torch.cuda.synchronize()
        g.replay()
        got = state()
        want = eager[r]
        if dispatch == ga.DISPATCH_MULTI:
            assert np.array_equal(got[0], want[0]), f"replay {r}: outputs differ from the eager calls"
        else:
            # the one-dispatch path sums in an order that may depend on arrival
            assert np.max(np.abs(got[0] - want[0])) <= 1e-5 * np.sqrt(np.mean(want[0] ** 2)), f"replay {r}"
        for l in range(NL):
            assert np.array_equal(got[1][l], want[1][l]) and np.array_equal(got[2][l], want[2][l]), f"replay {r}"
            assert np.array_equal(got[3][l], np.asarray(lens) + n) and np.array_equal(got[3][l], want[3][l])
            assert got[4][l] == want[4][l] == 0
        if r == 0:
            ref = oracle_cache(*caches[0], lens, dtype)
            xb = _inputs(0, B, n, dtype)[0]
            if n == 1:
                w = oracle.decode(layers[0].ocfg, layers[0].ref, ref, xb[:, 0])
                e = rel_err(got[0][0, :, 0], w)
            else:
                w = oracle.verify(layers[0].ocfg, layers[0].ref, ref, xb)
                e = rel_err(got[0][0], w)
            assert e < TOL[dtype], f"replay 0 vs oracle: {e:.3e}"
    del g
