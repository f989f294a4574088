"""fp64 CPU oracle of the decoder attention block (test infrastructure only)."""
from .attn_block import (BF16, F16, STATUS_CAPACITY, STATUS_CROP_GROW, BlockConfig, KVCache,
                         LayerWeights, decode, kv_append, kv_crop, rms_norm, rne16, rope,
                         rope_frequencies, verify, widen)
