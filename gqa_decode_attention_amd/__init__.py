"""MI355X-native decoder attention block (gfx950 HIP kernels behind a C ABI).

The Python side only marshals arguments into ``libasr_attn.so``; see
``include/asr_attn.h`` for the contract of every entry point.
"""
from ._lib import (BF16, FP8_E4M3, DISPATCH_AUTO, DISPATCH_FUSED, DISPATCH_MULTI, EXPORTED, F16, F32, LIB_PATH,
                   STATUS_BAD_PAGE, STATUS_BAD_SLOT, STATUS_CAPACITY, PhaseEvents, STATUS_CROP_GROW, STATUS_SYNC_TIMEOUT, AsrAttnConfig,
                   AsrError, KVLayer, Weights, alloc_workspace, config, kv_append, kv_crop, layer_decode, layer_decode_noalloc, NOALLOC_SCRATCH_BYTES,
                   layer_verify, load, torch_dtype, workspace_bytes, AsrMlpConfig, MlpWeights, mlp_config,
                   mlp_workspace_bytes, mlp_layer, decoder_layer_workspace, decoder_layer_decode,
                   decoder_layer_verify, decoder_layer_mixed, layer_mixed, head_config, embed, lm_head_workspace, lm_head_argmax, accept_greedy, accept_greedy_mixed, next_block_len, recycle_draft)
