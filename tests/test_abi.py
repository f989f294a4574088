"""The C ABI library on the CPU: it loads, exports every declared entry point, and its
host-side validation answers without touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "asr_attn.h")


def _lib():
    import gqa_decode_attention_amd as ga
    if not os.path.exists(ga.LIB_PATH):
        from gqa_decode_attention_amd.build import build
        build()
    return ga, ga.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(asr_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    ga, lib = _lib()
    names = declared_functions()
    assert set(names) == set(ga.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", ga.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (asr_\w+)", out))
    for n in names:
        assert n in exported and hasattr(lib, n)


def test_library_carries_gfx950_code_objects():
    ga, _ = _lib()
    blob = open(ga.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_workspace_bytes_and_strerror():
    ga, lib = _lib()
    cfg = ga.config()
    n1 = ga.workspace_bytes(cfg, 1, 1024)
    n64 = ga.workspace_bytes(cfg, 64, 4112)
    assert 0 < n1 < n64
    bad = ga.config(head_dim=64)
    assert lib.asr_attn_workspace_bytes(ctypes.byref(bad), 1, 1024) == 0
    assert lib.asr_attn_workspace_bytes(ctypes.byref(cfg), 4096, 1024) == 0
    assert lib.asr_strerror(-3) == b"cache capacity exceeded (host lengths)"


def test_host_validation_without_gpu():
    ga, lib = _lib()
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced on the host
    w = ga._lib.AsrAttnWeights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    kv = ga._lib.AsrKvLayer(0x1000, 0x1000, 0x1000, None, 4, 64, 8, 128, ga.F16)
    cfg = ga.config()
    dec = lib.asr_attn_layer_decode
    args = lambda c, B: (ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), fake, None, None, B, None, None,
                         fake, fake, 1 << 30, None)
    assert dec(*args(cfg, 0)) == 0                              # B = 0: a no-op
    assert dec(*args(cfg, -1)) == -1
    assert dec(*args(ga.config(n_q_heads=12), 1)) == -1         # nq % nkv
    assert dec(*args(ga.config(n_q_heads=24, n_kv_heads=8), 1)) == -2   # group 3
    assert dec(*args(ga.config(hidden=1000), 1)) == -2
    assert dec(*args(ga.config(dtype="f16", out_dtype="bf16"), 1)) == -2
    assert dec(*args(ga.config(kv_split=20), 1)) == -1
    assert dec(*args(cfg, 5)) == -1                             # B > batch_cap without slots
    small = (ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, None, None, 1, None, None,
             fake, fake, 16, None)
    assert dec(*small) == -4
    hl = (ctypes.c_int32 * 1)(64)
    cap = (ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, None, None, 1,
           ctypes.cast(hl, P), None, fake, fake, 1 << 30, None)
    assert dec(*cap) == -3
    ver = lib.asr_attn_layer_verify
    assert ver(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, None, None, 1, 33, None, None,
               fake, fake, 1 << 30, None) == -1
    assert lib.asr_kv_crop(None, 1, fake, None) == -1
    assert lib.asr_kv_crop(None, 0, None, None) == 0
    assert lib.asr_kv_append(ctypes.byref(kv), fake, fake, None, 0, 3, None) == 0
