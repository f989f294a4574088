"""MI355X-native decoder attention block (gfx950 HIP kernels behind a C ABI).

The Python side only marshals arguments into ``libasr_attn.so``; see
``include/asr_attn.h`` for the contract of every entry point.
"""
from ._lib import (BF16, DISPATCH_AUTO, DISPATCH_FUSED, DISPATCH_MULTI, EXPORTED, F16, F32, LIB_PATH,
                   STATUS_BAD_SLOT, STATUS_CAPACITY, PhaseEvents, STATUS_CROP_GROW, STATUS_SYNC_TIMEOUT, AsrAttnConfig,
                   AsrError, KVLayer, Weights, alloc_workspace, config, kv_append, kv_crop, layer_decode,
                   layer_verify, load, torch_dtype, workspace_bytes)
