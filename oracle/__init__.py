"""fp64 CPU oracle of the decoder attention block (test infrastructure only)."""
from .attn_block import (BF16, E4M3, E4M3_MAX, F16, e4m3_value, rne_e4m3, STATUS_CAPACITY, STATUS_CROP_GROW, BlockConfig, KVCache,
                         LayerWeights, decode, kv_append, kv_crop, mixed, rms_norm, rne16, rope,
                         rope_frequencies, verify, widen)
from .decoder_layer import MlpConfig, MlpWeights, decoder_layer_decode, decoder_layer_mixed, decoder_layer_verify, mlp, silu
from .spec_loop import (HeadConfig, TinyModel, accept_greedy, argmax_first, embed, greedy_decode, lm_head_logits,
                        speculative_round)
from .spec_policy import next_block_len, recycle_draft, speculative_decode
from .paged_kv import STATUS_BAD_PAGE, PagedKV, on_pages
