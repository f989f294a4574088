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

F16, BF16, F32 = 0, 1, 2
DISPATCH_AUTO, DISPATCH_MULTI, DISPATCH_FUSED = 0, 1, 2
STATUS_CAPACITY, STATUS_CROP_GROW, STATUS_SYNC_TIMEOUT, STATUS_BAD_SLOT = 1, 2, 4, 8

ERRORS = {0: "ASR_OK", -1: "ASR_EINVAL", -2: "ASR_EUNSUPPORTED", -3: "ASR_ECAPACITY",
          -4: "ASR_EWORKSPACE", -5: "ASR_EHIP"}

EXPORTED = ["asr_attn_workspace_bytes", "asr_attn_layer_decode", "asr_attn_layer_verify",
            "asr_kv_append", "asr_kv_crop", "asr_strerror"]

_TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}
_DT_NAME = {"f16": F16, "bf16": BF16, "f32": F32}


class AsrAttnConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("kv_split", ctypes.c_int32), ("dispatch", ctypes.c_int32),
                ("phase_events", ctypes.c_void_p)]


class AsrAttnWeights(ctypes.Structure):
    _fields_ = [("input_norm_w", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p)]


class AsrKvLayer(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("lens", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("batch_cap", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


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
    lib.asr_attn_layer_verify.argtypes = [ctypes.POINTER(AsrAttnConfig), ctypes.POINTER(AsrAttnWeights),
                                          ctypes.POINTER(AsrKvLayer), P, P, P, I32, I32, P, P, P, P, SZ, P]
    lib.asr_attn_layer_verify.restype = ctypes.c_int
    lib.asr_kv_append.argtypes = [ctypes.POINTER(AsrKvLayer), P, P, P, I32, I32, P]
    lib.asr_kv_append.restype = ctypes.c_int
    lib.asr_kv_crop.argtypes = [ctypes.POINTER(AsrKvLayer), I32, P, P]
    lib.asr_kv_crop.restype = ctypes.c_int
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
           dtype="f16", out_dtype="f32", kv_split=0, dispatch=DISPATCH_AUTO) -> AsrAttnConfig:
    return AsrAttnConfig(hidden, n_q_heads, n_kv_heads, head_dim, rms_eps, rope_theta,
                         _dt(dtype), _dt(out_dtype), kv_split, dispatch, None)


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
    """One layer's cache: k, v [batch_cap][nkv][capacity][d], lens [batch_cap] int32, status [1] int32."""

    def __init__(self, k, v, lens, status=None):
        assert k.shape == v.shape and k.dim() == 4 and k.dtype == v.dtype
        assert lens.dtype == torch.int32 and lens.numel() == k.shape[0]
        self.k, self.v, self.lens, self.status = k, v, lens, status
        dt = {torch.float16: F16, torch.bfloat16: BF16}[k.dtype]
        self.c = AsrKvLayer(k.data_ptr(), v.data_ptr(), lens.data_ptr(),
                            None if status is None else status.data_ptr(),
                            k.shape[0], k.shape[2], k.shape[1], k.shape[3], dt)

    @classmethod
    def empty(cls, batch_cap, n_kv_heads, capacity, head_dim=128, dtype=torch.float16, device="cuda"):
        shape = (batch_cap, n_kv_heads, capacity, head_dim)
        return cls(torch.zeros(shape, dtype=dtype, device=device), torch.zeros(shape, dtype=dtype, device=device),
                   torch.zeros(batch_cap, dtype=torch.int32, device=device),
                   torch.zeros(1, dtype=torch.int32, device=device))


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


def layer_verify(cfg, w: Weights, kv: KVLayer, x, out, workspace, slots=None, positions=None,
                 host_lens=None, residual=None, stream=None) -> None:
    keep, hl = _host_lens(host_lens)
    B, k = x.shape[0], x.shape[1]
    _check(load().asr_attn_layer_verify(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(kv.c), _ptr(x),
                                        _ptr(slots), _ptr(positions), B, k, hl, _ptr(residual), _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(stream)),
           "asr_attn_layer_verify")
    del keep


def kv_append(kv: KVLayer, k_new, v_new, slots=None, stream=None) -> None:
    B, n = k_new.shape[0], k_new.shape[1]
    _check(load().asr_kv_append(ctypes.byref(kv.c), _ptr(k_new), _ptr(v_new), _ptr(slots), B, n,
                                _stream(stream)), "asr_kv_append")


def kv_crop(layers, new_lens, stream=None) -> None:
    arr = (AsrKvLayer * len(layers))(*[l.c for l in layers])
    _check(load().asr_kv_crop(arr, len(layers), _ptr(new_lens), _stream(stream)), "asr_kv_crop")
