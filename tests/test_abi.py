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


def test_noalloc_entry_validates_on_the_host():
    """The workspace-free decode rejects, before touching a GPU, a call whose workspace would
    exceed its static scratch (ASR_ESCRATCH), and answers like the decode entry otherwise."""
    ga, lib = _lib()
    fake = ctypes.c_void_p(0x1000)
    w = ga._lib.AsrAttnWeights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    kv = ga._lib.AsrKvLayer(0x1000, 0x1000, 0x1000, None, 128, 1536, 8, 128, ga.BF16)
    cfg = ga.config(dtype="bf16")
    dec = lib.asr_attn_layer_decode_noalloc
    args = lambda c, B: (ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), fake, None, None, B, None, None, fake,
                         None)
    assert ga.workspace_bytes(cfg, 64, 1536) <= ga.NOALLOC_SCRATCH_BYTES < ga.workspace_bytes(cfg, 80, 1536)
    assert dec(*args(cfg, 80)) == -6
    assert lib.asr_strerror(-6).startswith(b"call needs more scratch")
    assert dec(*args(cfg, 0)) == 0
    assert dec(*args(cfg, -1)) == -1
    assert dec(*args(ga.config(hidden=1000, dtype="bf16"), 1)) == -2
    assert dec(*args(ga.config(head_dim=64, dtype="bf16"), 1)) == -2


def test_workspace_counters_sit_at_fixed_offsets():
    """Calls of different row counts may share one workspace: the counters every call leaves at
    zero come first, so a workspace sized for many rows holds a small call's data only after
    them (the bytes needed grow with the rows by the per-row regions alone)."""
    ga, _ = _lib()
    cfg = ga.config()
    n1, n2, n3 = (ga.workspace_bytes(cfg, r, 1024) for r in (1, 2, 3))
    assert n1 > 2048 * 32 * 4            # the counter block of the largest call is always there
    assert abs((n3 - n2) - (n2 - n1)) <= 8 * 256   # per-row regions only (256-byte alignment)


def test_fp8_cache_validation_on_the_host():
    """An FP8 cache needs its K and V scales; it takes calls of more than 4 rows only."""
    ga, lib = _lib()
    fake = ctypes.c_void_p(0x1000)
    w = ga._lib.AsrAttnWeights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cfg = ga.config(dtype="bf16")
    no_scales = ga._lib.AsrKvLayer(0x1000, 0x1000, 0x1000, None, 8, 64, 8, 128, ga.FP8_E4M3, None, None)
    scaled = ga._lib.AsrKvLayer(0x1000, 0x1000, 0x1000, None, 8, 64, 8, 128, ga.FP8_E4M3, 0x1000, 0x1000)
    dec = lib.asr_attn_layer_decode
    args = lambda kv, B, c=cfg: (ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), fake, None, None, B, None, None,
                                 fake, fake, 1 << 30, None)
    assert dec(*args(no_scales, 6)) == -1
    assert dec(*args(scaled, 4)) == -2                               # few rows: no FP8 kernel
    assert dec(*args(scaled, 6, ga.config(dtype="bf16", n_kv_heads=2)), ) == -1   # kv heads differ from the cache
    assert dec(*args(scaled, 6, ga.config(dtype="bf16", dispatch=ga.DISPATCH_FUSED))) == -2
    assert lib.asr_kv_append(ctypes.byref(no_scales), fake, fake, None, 1, 1, None) == -1


def test_mixed_entry_validates_on_the_host():
    """Mixed calls: block sizes 1 .. 32 for at most 64 sequences, no fused dispatch, the host
    lengths checked against each sequence's own block."""
    ga, lib = _lib()
    P = ctypes.c_void_p
    fake = P(0x1000)
    w = ga._lib.AsrAttnWeights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    kv = ga._lib.AsrKvLayer(0x1000, 0x1000, 0x1000, None, 80, 64, 8, 128, ga.F16)
    cfg = ga.config()
    mix = lib.asr_attn_layer_mixed

    def call(sizes, c=cfg, lens=None, ws=1 << 30):
        nb = (ctypes.c_int32 * max(1, len(sizes)))(*sizes)
        hl = None if lens is None else ctypes.cast((ctypes.c_int32 * len(lens))(*lens), P)
        return mix(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), fake, None, None, len(sizes),
                   ctypes.cast(nb, P), hl, None, fake, fake, ws, None)

    assert call([]) == 0
    assert mix(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, None, None, 2, None, None, None, fake,
               fake, 1 << 30, None) == -1                             # no block sizes
    assert call([1, 0, 2]) == -1 and call([33]) == -1 and call([1] * 65) == -1
    assert call([4, 1], ga.config(dispatch=ga.DISPATCH_FUSED)) == -2
    assert call([4, 8], lens=[60, 57]) == -3                          # 57 + 8 > 64
    assert call([4, 8], ws=16) == -4
    assert call([32] * 64, ws=16) == -4                               # the largest call: 2048 rows


def test_paged_cache_validation_on_the_host():
    """A paged cache: power-of-two pages of 16 .. 1024 rows, capacity = pages_per_seq * page_size,
    a non-empty pool, 16-bit elements, the stream-ordered dispatch; the prefill copy checks the
    same descriptor."""
    ga, lib = _lib()
    fake = ctypes.c_void_p(0x1000)
    w = ga._lib.AsrAttnWeights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cfg = ga.config()

    def kv(page=16, pps=4, cap=None, num=32, dt=ga.F16, scales=(None, None)):
        cap = page * pps if cap is None else cap
        return ga._lib.AsrKvLayer(0x1000, 0x1000, 0x1000, None, 8, cap, 8, 128, dt, *scales, 0x1000, page, pps, num)

    dec = lib.asr_attn_layer_decode
    args = lambda c_kv, B=1, c=cfg, ws=1 << 30: (ctypes.byref(c), ctypes.byref(w), ctypes.byref(c_kv), fake, None,
                                                 None, B, None, None, fake, fake, ws, None)
    assert dec(*args(kv(page=24, pps=4))) == -2                    # not a power of two
    assert dec(*args(kv(page=8, pps=8))) == -2                     # below 16 rows
    assert dec(*args(kv(page=2048, pps=1))) == -2                  # above 1024 rows
    assert dec(*args(kv(cap=100))) == -1                           # capacity != pages_per_seq * page_size
    assert dec(*args(kv(num=0))) == -1
    assert dec(*args(kv(pps=0, cap=16))) == -1
    assert dec(*args(kv(dt=ga.FP8_E4M3, scales=(0x1000, 0x1000)), 6, ga.config(dtype="bf16"))) == -2
    assert dec(*args(kv(), 1, ga.config(dispatch=ga.DISPATCH_FUSED))) == -2
    assert dec(*args(kv(), 0)) == 0
    assert dec(*args(kv(), 1, cfg, 16)) == -4                      # the workspace check still applies
    assert lib.asr_kv_append(ctypes.byref(kv(page=48)), fake, fake, None, 1, 1, None) == -2
    assert lib.asr_kv_append(ctypes.byref(kv()), fake, fake, None, 0, 1, None) == 0
    # the descriptor's layout: the paged fields follow the FP8 scales
    assert ctypes.sizeof(ga._lib.AsrKvLayer) == 96
    assert ga._lib.AsrKvLayer.block_table.offset == 72 and ga._lib.AsrKvLayer.num_pages.offset == 88
