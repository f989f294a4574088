"""The benchmark's byte model and command-line contract (CPU).

The roofline fraction divides algorithmic bytes by a measured duration, so
the byte model is pinned here against sizes fixed by the block's shapes:
per layer at hidden 1024 the weights are 4096 x 1024 (W_qkv) + 1024 x 2048
(W_o) + 1024 + 2 x 128 (gains) 16-bit elements, and each cached position
holds K and V for 8 heads of 128 16-bit values.
"""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_layer_weight_bytes():
    b = _bench()
    p = b.phase_bytes(1024, 16, 8, 128, [0], 0)   # no rows, no cache: weights and gains only
    assert p["qkv_projection"] + p["o_proj"] == 12_585_472
    p = b.phase_bytes(2048, 16, 8, 128, [0], 0)
    assert p["qkv_projection"] + p["o_proj"] == 25_170_432


def test_cache_and_activation_bytes():
    b = _bench()
    # bs1 decode at committed length 795: K and V read once (4096 B per position), the new row written
    p = b.phase_bytes(1024, 16, 8, 128, [795], 1)
    assert p["attention"] == 795 * 4096 + 4096
    assert p["qkv_projection"] == (4096 * 1024 + 1024 + 256) * 2 + 1024 * 2   # + x, 16-bit
    assert p["o_proj"] == 1024 * 2048 * 2 + 1024 * 4                          # + out, fp32
    # ragged rows add up
    lens = [200, 1500, 777]
    assert b.phase_bytes(1024, 16, 8, 128, lens, 3)["attention"] == sum(lens) * 4096 + 3 * 4096
    assert b.layer_bytes(1024, 16, 8, 128, [795], 1) == sum(b.phase_bytes(1024, 16, 8, 128, [795], 1).values())


def test_roofline_picks_the_longest_kernel():
    b = _bench()
    mean_us = {"qkv_projection": 4.0, "attention": 6.0, "o_proj": 4.5}
    bphase = {"qkv_projection": 8e6, "attention": 3.0e6, "o_proj": 4e6}
    r = b.roofline(mean_us, bphase, {"attention": 123})
    assert r["kernel"] == "attention" and r["traffic"] == 123
    assert abs(r["achieved"] - 3.0e6 / 6e-6 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    assert b.roofline(mean_us, bphase, None)["traffic"] is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_fp8_cache_halves_the_cache_bytes_only():
    b = _bench()
    p16 = b.phase_bytes(1024, 16, 8, 128, [200, 1500], 2)
    p8 = b.phase_bytes(1024, 16, 8, 128, [200, 1500], 2, e_kv=1)
    assert p8["attention"] * 2 == p16["attention"]
    assert p8["qkv_projection"] == p16["qkv_projection"] and p8["o_proj"] == p16["o_proj"]


def test_step_roofline_is_bytes_over_time():
    b = _bench()
    r = b.step_roofline(8e9, 1.0)        # 8 GB in 1 ms = 8000 GB/s
    assert r["achieved"] == 8000.0 and r["frac"] == 1.0 and r["unit"] == "GB/s"
