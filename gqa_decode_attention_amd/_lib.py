"""ctypes binding of libasr_attn.so: argument marshalling only.

Every computation runs in the HIP library.  Tensors are PyTorch tensors on
the GPU; their device pointers and torch's current HIP stream are passed
through unchanged.  If the library has not been built, loading raises: there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime first; the library binds to that one)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libasr_attn.so")

F16, BF16, F32, FP8_E4M3 = 0, 1, 2, 3
DISPATCH_AUTO, DISPATCH_MULTI, DISPATCH_FUSED = 0, 1, 2
STATUS_CAPACITY, STATUS_CROP_GROW, STATUS_SYNC_TIMEOUT, STATUS_BAD_SLOT, STATUS_BAD_PAGE = 1, 2, 4, 8, 16

ERRORS = {0: "ASR_OK", -1: "ASR_EINVAL", -2: "ASR_EUNSUPPORTED", -3: "ASR_ECAPACITY",
          -4: "ASR_EWORKSPACE", -5: "ASR_EHIP", -6: "ASR_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 40 << 20

EXPORTED = ["asr_attn_workspace_bytes", "asr_attn_layer_decode", "asr_attn_layer_decode_noalloc",
            "asr_attn_layer_verify", "asr_kv_append", "asr_kv_crop", "asr_strerror",
            "asr_mlp_workspace_bytes", "asr_mlp_layer", "asr_decoder_layer_workspace_bytes",
            "asr_decoder_layer_decode", "asr_decoder_layer_verify", "asr_embed", "asr_lm_head_workspace_bytes",
            "asr_lm_head_argmax", "asr_accept_greedy", "asr_attn_layer_mixed", "asr_decoder_layer_mixed",
            "asr_accept_greedy_mixed", "asr_next_block_len", "asr_recycle_draft"]

_TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}
_DT_NAME = {"f16": F16, "bf16": BF16, "f32": F32}


class AsrAttnConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("kv_split", ctypes.c_int32), ("dispatch", ctypes.c_int32),
                ("phase_events", ctypes.c_void_p), ("mrope_sections", ctypes.c_int32 * 3)]


class AsrAttnWeights(ctypes.Structure):
    _fields_ = [("input_norm_w", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p)]


class AsrKvLayer(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("lens", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("batch_cap", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class AsrMlpConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("phase_events", ctypes.c_void_p)]


class AsrMlpWeights(ctypes.Structure):
    _fields_ = [("post_norm_w", ctypes.c_void_p), ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


class AsrHeadConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("in_dtype", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m gqa_decode_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.asr_attn_workspace_bytes.argtypes = [ctypes.POINTER(AsrAttnConfig), I32, I32]
    lib.asr_attn_workspace_bytes.restype = SZ
    lib.asr_attn_layer_decode.argtypes = [ctypes.POINTER(AsrAttnConfig), ctypes.POINTER(AsrAttnWeights),
                                          ctypes.POINTER(AsrKvLayer), P, P, P, I32, P, P, P, P, SZ, P]
    lib.asr_attn_layer_decode.restype = ctypes.c_int
    lib.asr_attn_layer_decode_noalloc.argtypes = [ctypes.POINTER(AsrAttnConfig), ctypes.POINTER(AsrAttnWeights),
                                                  ctypes.POINTER(AsrKvLayer), P, P, P, I32, P, P, P, P]
    lib.asr_attn_layer_decode_noalloc.restype = ctypes.c_int
    lib.asr_attn_layer_verify.argtypes = [ctypes.POINTER(AsrAttnConfig), ctypes.POINTER(AsrAttnWeights),
                                          ctypes.POINTER(AsrKvLayer), P, P, P, I32, I32, P, P, P, P, SZ, P]
    lib.asr_attn_layer_verify.restype = ctypes.c_int
    lib.asr_kv_append.argtypes = [ctypes.POINTER(AsrKvLayer), P, P, P, I32, I32, P]
    lib.asr_kv_append.restype = ctypes.c_int
    lib.asr_kv_crop.argtypes = [ctypes.POINTER(AsrKvLayer), I32, P, P]
    lib.asr_kv_crop.restype = ctypes.c_int
    MC, MW, AC, AW, KV = (ctypes.POINTER(AsrMlpConfig), ctypes.POINTER(AsrMlpWeights), ctypes.POINTER(AsrAttnConfig),
                          ctypes.POINTER(AsrAttnWeights), ctypes.POINTER(AsrKvLayer))
    lib.asr_mlp_workspace_bytes.argtypes = [MC, I32]
    lib.asr_mlp_workspace_bytes.restype = SZ
    lib.asr_mlp_layer.argtypes = [MC, MW, P, I32, P, P, SZ, P]
    lib.asr_mlp_layer.restype = ctypes.c_int
    lib.asr_decoder_layer_workspace_bytes.argtypes = [AC, MC, I32, I32]
    lib.asr_decoder_layer_workspace_bytes.restype = SZ
    lib.asr_decoder_layer_decode.argtypes = [AC, AW, MC, MW, KV, P, P, P, I32, P, P, P, SZ, P]
    lib.asr_decoder_layer_decode.restype = ctypes.c_int
    lib.asr_decoder_layer_verify.argtypes = [AC, AW, MC, MW, KV, P, P, P, I32, I32, P, P, P, SZ, P]
    lib.asr_decoder_layer_verify.restype = ctypes.c_int
    lib.asr_attn_layer_mixed.argtypes = [AC, AW, KV, P, P, P, I32, P, P, P, P, P, SZ, P]
    lib.asr_attn_layer_mixed.restype = ctypes.c_int
    lib.asr_decoder_layer_mixed.argtypes = [AC, AW, MC, MW, KV, P, P, P, I32, P, P, P, P, SZ, P]
    lib.asr_decoder_layer_mixed.restype = ctypes.c_int
    lib.asr_accept_greedy_mixed.argtypes = [P, P, I32, P, P, P, I32, P, P, P, P]
    lib.asr_accept_greedy_mixed.restype = ctypes.c_int
    lib.asr_next_block_len.argtypes = [P, I32, ctypes.c_float, I32, I32]
    lib.asr_next_block_len.restype = ctypes.c_int32
    lib.asr_recycle_draft.argtypes = [P, I32, I32, I32, I32, I32, I32]
    lib.asr_recycle_draft.restype = ctypes.c_int32
    HC = ctypes.POINTER(AsrHeadConfig)
    lib.asr_embed.argtypes = [P, I32, I32, I32, P, I32, P, P]
    lib.asr_embed.restype = ctypes.c_int
    lib.asr_lm_head_workspace_bytes.argtypes = [HC, I32]
    lib.asr_lm_head_workspace_bytes.restype = SZ
    lib.asr_lm_head_argmax.argtypes = [HC, P, P, P, I32, P, P, P, SZ, P]
    lib.asr_lm_head_argmax.restype = ctypes.c_int
    lib.asr_accept_greedy.argtypes = [P, P, I32, I32, P, P, I32, P, P, P, P]
    lib.asr_accept_greedy.restype = ctypes.c_int
    lib.asr_strerror.argtypes = [ctypes.c_int]
    lib.asr_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


class AsrError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = load().asr_strerror(code).decode()
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({msg})")


def _check(code: int, what: str) -> None:
    if code != 0:
        raise AsrError(code, what)


def _dt(x) -> int:
    return _DT_NAME[x] if isinstance(x, str) else int(x)


def torch_dtype(dt) -> torch.dtype:
    return _TORCH_DT[_dt(dt)]


def config(hidden=1024, n_q_heads=16, n_kv_heads=8, head_dim=128, rms_eps=1e-6, rope_theta=1e6,
           dtype="f16", out_dtype="f32", kv_split=0, dispatch=DISPATCH_AUTO, mrope_sections=(0, 0, 0)) -> AsrAttnConfig:
    return AsrAttnConfig(hidden, n_q_heads, n_kv_heads, head_dim, rms_eps, rope_theta,
                         _dt(dtype), _dt(out_dtype), kv_split, dispatch, None,
                         (ctypes.c_int32 * 3)(*mrope_sections))


class PhaseEvents:
    """Six torch.cuda.Events that receive the start and end stamps of a layer call's three phase
    kernels (diagnostics).  Attach with ``cfg.phase_events = pe.ptr``; read with ``elapsed_ms()``."""

    def __init__(self):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in self.events:   # materialise the underlying hipEvent_t handles
            e.record()
        self._arr = (ctypes.c_void_p * 6)(*[e.cuda_event for e in self.events])
        self.ptr = ctypes.cast(self._arr, ctypes.c_void_p)

    def elapsed_ms(self):
        """(projection, attention, o_proj) kernel durations of the last call, in ms."""
        ev = self.events
        return tuple(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(3))

    def total_ms(self):
        """First kernel start to last kernel end of the last call, in ms (also for the fused dispatch)."""
        return self.events[0].elapsed_time(self.events[5])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Weights:
    """One layer's weights as device tensors (16-bit)."""

    def __init__(self, input_norm_w, w_qkv, q_norm_w, k_norm_w, w_o):
        self.input_norm_w, self.w_qkv, self.q_norm_w = input_norm_w, w_qkv, q_norm_w
        self.k_norm_w, self.w_o = k_norm_w, w_o
        self.c = AsrAttnWeights(*(t.data_ptr() for t in (input_norm_w, w_qkv, q_norm_w, k_norm_w, w_o)))


class KVLayer:
    """One layer's cache: k, v [batch_cap][nkv][capacity][d], lens [batch_cap] int32, status [1] int32.

    16-bit caches are float16 / bfloat16 tensors; an FP8 cache is uint8 tensors of E4M3 codes
    with fp32 per-kv-head scales ``k_scale``, ``v_scale`` [nkv] on the device.  A paged cache
    (``block_table`` [batch_cap][pages_per_seq] int32 on the device) has pools
    k, v [num_pages][nkv][page_size][d] instead."""

    def __init__(self, k, v, lens, status=None, k_scale=None, v_scale=None, block_table=None):
        assert k.shape == v.shape and k.dim() == 4 and k.dtype == v.dtype
        assert lens.dtype == torch.int32
        self.k, self.v, self.lens, self.status = k, v, lens, status
        self.k_scale, self.v_scale, self.block_table = k_scale, v_scale, block_table
        dt = {torch.float16: F16, torch.bfloat16: BF16, torch.uint8: FP8_E4M3}[k.dtype]
        if dt == FP8_E4M3:
            assert k_scale is not None and v_scale is not None
            assert k_scale.dtype == torch.float32 and v_scale.dtype == torch.float32
        if block_table is None:
            assert lens.numel() == k.shape[0]
            batch_cap, capacity, paged = k.shape[0], k.shape[2], (None, 0, 0, 0)
        else:
            assert block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
            assert lens.numel() == block_table.shape[0]
            batch_cap, pps = block_table.shape
            capacity = pps * k.shape[2]
            paged = (block_table.data_ptr(), k.shape[2], pps, k.shape[0])
        self.c = AsrKvLayer(k.data_ptr(), v.data_ptr(), lens.data_ptr(),
                            None if status is None else status.data_ptr(),
                            batch_cap, capacity, k.shape[1], k.shape[3], dt,
                            None if k_scale is None else k_scale.data_ptr(),
                            None if v_scale is None else v_scale.data_ptr(), *paged)

    @property
    def batch_cap(self) -> int:
        return self.c.batch_cap

    @property
    def capacity(self) -> int:
        return self.c.capacity

    @classmethod
    def empty(cls, batch_cap, n_kv_heads, capacity, head_dim=128, dtype=torch.float16, device="cuda",
              k_scale=None, v_scale=None):
        shape = (batch_cap, n_kv_heads, capacity, head_dim)
        return cls(torch.zeros(shape, dtype=dtype, device=device), torch.zeros(shape, dtype=dtype, device=device),
                   torch.zeros(batch_cap, dtype=torch.int32, device=device),
                   torch.zeros(1, dtype=torch.int32, device=device), k_scale, v_scale)

    @classmethod
    def paged(cls, num_pages, n_kv_heads, page_size, block_table, head_dim=128, dtype=torch.float16,
              device="cuda"):
        """A zeroed pool of num_pages pages and the given page table [batch_cap][pages_per_seq]."""
        shape = (num_pages, n_kv_heads, page_size, head_dim)
        bt = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        return cls(torch.zeros(shape, dtype=dtype, device=device), torch.zeros(shape, dtype=dtype, device=device),
                   torch.zeros(bt.shape[0], dtype=torch.int32, device=device),
                   torch.zeros(1, dtype=torch.int32, device=device), block_table=bt)


def workspace_bytes(cfg: AsrAttnConfig, max_rows: int, capacity: int) -> int:
    n = load().asr_attn_workspace_bytes(ctypes.byref(cfg), max_rows, capacity)
    if n == 0:
        raise AsrError(-1, "asr_attn_workspace_bytes")
    return int(n)


def alloc_workspace(cfg: AsrAttnConfig, max_rows: int, capacity: int, device="cuda") -> torch.Tensor:
    return torch.zeros(workspace_bytes(cfg, max_rows, capacity), dtype=torch.uint8, device=device)


def _host_lens(host_lens):
    if host_lens is None:
        return None, None
    arr = (ctypes.c_int32 * len(host_lens))(*[int(v) for v in host_lens])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def layer_decode(cfg, w: Weights, kv: KVLayer, x, out, workspace, slots=None, positions=None,
                 host_lens=None, residual=None, stream=None) -> None:
    keep, hl = _host_lens(host_lens)
    B = x.shape[0]
    _check(load().asr_attn_layer_decode(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(kv.c), _ptr(x),
                                        _ptr(slots), _ptr(positions), B, hl, _ptr(residual), _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(stream)),
           "asr_attn_layer_decode")
    del keep


def layer_decode_noalloc(cfg, w: Weights, kv: KVLayer, x, out, slots=None, positions=None,
                         host_lens=None, residual=None, stream=None) -> None:
    """layer_decode with the library's static per-GPU scratch instead of a workspace."""
    keep, hl = _host_lens(host_lens)
    B = x.shape[0]
    _check(load().asr_attn_layer_decode_noalloc(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(kv.c), _ptr(x),
                                                _ptr(slots), _ptr(positions), B, hl, _ptr(residual), _ptr(out),
                                                _stream(stream)),
           "asr_attn_layer_decode_noalloc")
    del keep


def layer_verify(cfg, w: Weights, kv: KVLayer, x, out, workspace, slots=None, positions=None,
                 host_lens=None, residual=None, stream=None) -> None:
    keep, hl = _host_lens(host_lens)
    B, k = x.shape[0], x.shape[1]
    _check(load().asr_attn_layer_verify(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(kv.c), _ptr(x),
                                        _ptr(slots), _ptr(positions), B, k, hl, _ptr(residual), _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(stream)),
           "asr_attn_layer_verify")
    del keep


def _block_sizes(n_per_seq):
    """HOST int32 array of the block sizes (a sequence of ints)."""
    sizes = [int(v) for v in n_per_seq]
    arr = (ctypes.c_int32 * max(1, len(sizes)))(*sizes)
    return arr, len(sizes)


def layer_mixed(cfg, w: Weights, kv: KVLayer, x, n_per_seq, out, workspace, slots=None, positions=None,
                host_lens=None, residual=None, stream=None) -> None:
    """Decode rows and verify blocks of per-sequence sizes n_per_seq (host ints) in one call:
    x, residual, out [sum(n_per_seq)][H]."""
    keep, hl = _host_lens(host_lens)
    nb, B = _block_sizes(n_per_seq)
    _check(load().asr_attn_layer_mixed(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(kv.c), _ptr(x),
                                       _ptr(slots), _ptr(positions), B, ctypes.cast(nb, ctypes.c_void_p), hl,
                                       _ptr(residual), _ptr(out), _ptr(workspace), workspace.numel(),
                                       _stream(stream)),
           "asr_attn_layer_mixed")
    del keep, nb


def kv_append(kv: KVLayer, k_new, v_new, slots=None, stream=None) -> None:
    B, n = k_new.shape[0], k_new.shape[1]
    _check(load().asr_kv_append(ctypes.byref(kv.c), _ptr(k_new), _ptr(v_new), _ptr(slots), B, n,
                                _stream(stream)), "asr_kv_append")


def kv_crop(layers, new_lens, stream=None) -> None:
    arr = (AsrKvLayer * len(layers))(*[l.c for l in layers])
    _check(load().asr_kv_crop(arr, len(layers), _ptr(new_lens), _stream(stream)), "asr_kv_crop")


def mlp_config(hidden=1024, intermediate=3072, rms_eps=1e-6, dtype="f16", in_dtype="f32", out_dtype="f32"):
    return AsrMlpConfig(hidden, intermediate, rms_eps, _dt(dtype), _dt(in_dtype), _dt(out_dtype), None)


class MlpWeights:
    """One layer's MLP weights as device tensors (16-bit): post-norm gain [H], gate and up [I][H], down [H][I]."""

    def __init__(self, post_norm_w, w_gate, w_up, w_down):
        self.post_norm_w, self.w_gate, self.w_up, self.w_down = post_norm_w, w_gate, w_up, w_down
        self.c = AsrMlpWeights(*(t.data_ptr() for t in (post_norm_w, w_gate, w_up, w_down)))


def mlp_workspace_bytes(cfg: AsrMlpConfig, max_rows: int) -> int:
    n = load().asr_mlp_workspace_bytes(ctypes.byref(cfg), max_rows)
    if n == 0:
        raise AsrError(-1, "asr_mlp_workspace_bytes")
    return int(n)


def mlp_layer(cfg, w: MlpWeights, h, out, workspace, stream=None) -> None:
    _check(load().asr_mlp_layer(ctypes.byref(cfg), ctypes.byref(w.c), _ptr(h), h.shape[0], _ptr(out),
                                _ptr(workspace), workspace.numel(), _stream(stream)), "asr_mlp_layer")


def decoder_layer_workspace(acfg, mcfg, max_rows: int, capacity: int, device="cuda") -> torch.Tensor:
    n = load().asr_decoder_layer_workspace_bytes(ctypes.byref(acfg), ctypes.byref(mcfg), max_rows, capacity)
    if n == 0:
        raise AsrError(-1, "asr_decoder_layer_workspace_bytes")
    return torch.zeros(int(n), dtype=torch.uint8, device=device)


def decoder_layer_decode(acfg, aw: Weights, mcfg, mw: MlpWeights, kv: KVLayer, x, out, workspace, slots=None,
                         positions=None, host_lens=None, stream=None) -> None:
    keep, hl = _host_lens(host_lens)
    _check(load().asr_decoder_layer_decode(ctypes.byref(acfg), ctypes.byref(aw.c), ctypes.byref(mcfg),
                                           ctypes.byref(mw.c), ctypes.byref(kv.c), _ptr(x), _ptr(slots),
                                           _ptr(positions), x.shape[0], hl, _ptr(out), _ptr(workspace),
                                           workspace.numel(), _stream(stream)), "asr_decoder_layer_decode")
    del keep


def decoder_layer_verify(acfg, aw: Weights, mcfg, mw: MlpWeights, kv: KVLayer, x, out, workspace, slots=None,
                         positions=None, host_lens=None, stream=None) -> None:
    keep, hl = _host_lens(host_lens)
    _check(load().asr_decoder_layer_verify(ctypes.byref(acfg), ctypes.byref(aw.c), ctypes.byref(mcfg),
                                           ctypes.byref(mw.c), ctypes.byref(kv.c), _ptr(x), _ptr(slots),
                                           _ptr(positions), x.shape[0], x.shape[1], hl, _ptr(out),
                                           _ptr(workspace), workspace.numel(), _stream(stream)),
           "asr_decoder_layer_verify")
    del keep


def decoder_layer_mixed(acfg, aw: Weights, mcfg, mw: MlpWeights, kv: KVLayer, x, n_per_seq, out, workspace,
                        slots=None, positions=None, host_lens=None, stream=None) -> None:
    keep, hl = _host_lens(host_lens)
    nb, B = _block_sizes(n_per_seq)
    _check(load().asr_decoder_layer_mixed(ctypes.byref(acfg), ctypes.byref(aw.c), ctypes.byref(mcfg),
                                          ctypes.byref(mw.c), ctypes.byref(kv.c), _ptr(x), _ptr(slots),
                                          _ptr(positions), B, ctypes.cast(nb, ctypes.c_void_p), hl, _ptr(out),
                                          _ptr(workspace), workspace.numel(), _stream(stream)),
           "asr_decoder_layer_mixed")
    del keep, nb


def head_config(hidden=1024, vocab=151936, rms_eps=1e-6, dtype="f16", in_dtype="f32"):
    return AsrHeadConfig(hidden, vocab, rms_eps, _dt(dtype), _dt(in_dtype))


def embed(table, ids, x, stream=None) -> None:
    """x[r] = table[ids[r]]; table [V][H] 16-bit, ids int32 [rows], x [rows][H]."""
    dt = {torch.float16: F16, torch.bfloat16: BF16}[table.dtype]
    _check(load().asr_embed(_ptr(table), table.shape[0], table.shape[1], dt, _ptr(ids), ids.numel(), _ptr(x),
                            _stream(stream)), "asr_embed")


def lm_head_workspace(cfg, max_rows: int, device="cuda") -> torch.Tensor:
    n = load().asr_lm_head_workspace_bytes(ctypes.byref(cfg), max_rows)
    if n == 0:
        raise AsrError(-1, "asr_lm_head_workspace_bytes")
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def lm_head_argmax(cfg, final_norm_w, w_lm, h, ids, workspace, max_logit=None, stream=None) -> None:
    _check(load().asr_lm_head_argmax(ctypes.byref(cfg), _ptr(final_norm_w), _ptr(w_lm), _ptr(h), h.shape[0],
                                     _ptr(ids), _ptr(max_logit), _ptr(workspace), workspace.numel(),
                                     _stream(stream)), "asr_lm_head_argmax")


def accept_greedy(draft, target, lens, accepted, next_token, new_lens, slots=None, stream=None) -> None:
    """draft, target int32 [B][k]; lens, new_lens int32 [batch_cap]; accepted, next_token int32 [B]."""
    B, k = draft.shape
    _check(load().asr_accept_greedy(_ptr(draft), _ptr(target), B, k, _ptr(slots), _ptr(lens), lens.numel(),
                                    _ptr(accepted), _ptr(next_token), _ptr(new_lens), _stream(stream)),
           "asr_accept_greedy")


def accept_greedy_mixed(draft, target, n_per_seq, lens, accepted, next_token, new_lens, slots=None,
                        stream=None) -> None:
    """draft, target int32 [sum(n_per_seq)] (sequence-major blocks); n_per_seq host ints."""
    nb, B = _block_sizes(n_per_seq)
    _check(load().asr_accept_greedy_mixed(_ptr(draft), _ptr(target), B, ctypes.cast(nb, ctypes.c_void_p),
                                          _ptr(slots), _ptr(lens), lens.numel(), _ptr(accepted), _ptr(next_token),
                                          _ptr(new_lens), _stream(stream)),
           "asr_accept_greedy_mixed")
    del nb


def next_block_len(uncertainty, threshold, k_min, k_max) -> int:
    """The next block length from the host uncertainties of the remaining draft tokens."""
    u = [float(v) for v in uncertainty]
    arr = (ctypes.c_float * max(1, len(u)))(*u)
    k = load().asr_next_block_len(ctypes.cast(arr, ctypes.c_void_p), len(u), float(threshold), int(k_min), int(k_max))
    _check(min(int(k), 0), "asr_next_block_len")
    return int(k)


def recycle_draft(draft, pos, k, accepted, correction, window) -> int:
    """The draft read position after a round (host token ids; correction ignored when all accepted)."""
    d = [int(v) for v in draft]
    arr = (ctypes.c_int32 * max(1, len(d)))(*d)
    p = load().asr_recycle_draft(ctypes.cast(arr, ctypes.c_void_p), len(d), int(pos), int(k), int(accepted),
                                 int(-1 if correction is None else correction), int(window))
    _check(min(int(p), 0), "asr_recycle_draft")
    return int(p)
