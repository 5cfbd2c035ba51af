"""MI355X-native sink-GQA attention: YaRN RoPE, append-only KV cache with
snapshot/restore, W-row ring caches for band layers, and sink attention for
prefill and decode on gfx950.

The compute lives in libsinkattn.so (hand-written HIP kernels behind a C
ABI, ``include/sinkattn.h``); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    KVCache, KVRing, SinkAttnError, Yarn, decode_workspace, decode_workspace_bytes, kv_cache_bytes,
    last_error, moe_dispatch, moe_layer, moe_route, moe_workspace_bytes, qkv_rope_append, qkv_workspace_bytes,
    sample_count_tokens, sample_params, sample_tokens, sample_workspace_bytes, sinkattn_decode, sinkattn_decode_noalloc, decode_scratch_bytes,
    sinkattn_decode_step,
    sinkattn_prefill,
    sinkattn_prefill_rope, v_blocked, v_cache_shape, v_rows,
    yarn_inv_freq, yarn_rope_apply, LIB_PATH, SA_BF16, SA_F32,
)
