"""The workspace-free decode entry point against the decode entry point, through the C ABI.

Two calls in a row share the library's static scratch, the second with fewer rows than the
first; each must compute what asr_attn_layer_decode computes on its own workspace (the same
kernels: identical bits), which the oracle checks as well."""
import numpy as np
import pytest
import torch

import gqa_decode_attention_amd as ga
import oracle
from synth import inputs as si

from gpu_common import TOL, SeededLayer, device_cache, fill_cache, oracle_cache, rel_err, tdt, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _call(entry, cfg, L, kv, xb, dtype, slots, ws=None):
    B, H = xb.shape
    out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    st = torch.tensor(slots, dtype=torch.int32, device="cuda")
    if entry == "noalloc":
        ga.layer_decode_noalloc(cfg, L.dev, kv, to_dev(xb, dtype), out, slots=st)
    else:
        ga.layer_decode(cfg, L.dev, kv, to_dev(xb, dtype), out, ws, slots=st)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", [si.BF16, si.F16])
def test_noalloc_decode_equals_decode_on_two_calls(dtype):
    """A 64-row call (matrix-core path) then a 3-row call (few-row path) on the same caches."""
    lens = [int(v) for v in si.kv_lengths(8, 64, 200, 1500)]
    cap = 1536
    L = SeededLayer(8, 0, 1024, dtype)
    kb, vb = fill_cache(8, 0, lens, cap, dtype)
    plan = [list(range(64)), [5, 63, 0]]
    res = {}
    for entry in ("decode", "noalloc"):
        kv = device_cache(kb, vb, lens, dtype)
        cfg = ga.config(dtype=dtype)
        ws = ga.alloc_workspace(cfg, 64, cap) if entry == "decode" else None
        outs = [_call(entry, cfg, L, kv, si.activations(8, 0, step, len(sl), 1024, dtype), dtype, sl, ws)
                for step, sl in enumerate(plan)]
        res[entry] = (outs, to_bits(kv.k), to_bits(kv.v), kv.lens.cpu().numpy(), kv.status.item())
    a, b = res["decode"], res["noalloc"]
    for oa, ob in zip(a[0], b[0]):
        assert np.array_equal(oa, ob)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])
    assert a[4] == b[4] == 0
    # and both calls match the oracle run from the same seeded inputs
    ref = oracle_cache(kb, vb, lens, dtype)
    for step, sl in enumerate(plan):
        want = oracle.decode(L.ocfg, L.ref, ref, si.activations(8, 0, step, len(sl), 1024, dtype), slots=sl)
        err = rel_err(b[0][step], want)
        print(f"noalloc {dtype}: call {step} ({len(sl)} rows) max|err|/rms = {err:.3e}")
        assert err < TOL[dtype]
    assert np.array_equal(ref.lens, b[3])
