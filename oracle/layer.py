"""One attention layer's hot path, prefill and decode -- oracle, test infrastructure.

Order of the steps ("MoE-Xtend" README: one-page pseudocode, ARCHITECTURE,
TOKEN STREAM (DECODE), KV CACHE): rotate Q and K at global positions
offset + t, append the rotated K and the unrotated V at the cache offset
(which advances it), then attend.  The queries of a chunk start at the offset
the cache had before the append, so a decode step's query at position p sees
its own freshly appended row p.  "Decode stores rotated K and unchanged V"
(GPT-OSS-Lite visual guide, Model Architecture).

Rotated Q and K are rounded once to the storage dtype, as the interface
stores them; attention is computed in fp64 on those stored values and the
caller rounds or compares its fp64 result.
"""
import numpy as np

from .attention import sink_attention
from .rounding import round_to
from .yarn import rope_apply


def prefill_layer(cache, q, k, v, sinks, window, sm_scale, inv_freq, conc,
                  dtype):
    """q [B,T,n_q,d], k/v [B,T,n_kv,d] raw (pre-RoPE) values of the storage
    dtype.  Returns (out fp64 [B,T,n_q,d], q_rot, k_rot) and appends to cache."""
    o = cache.offset
    q_rot = round_to(rope_apply(q, o, inv_freq, conc), dtype)
    k_rot = round_to(rope_apply(k, o, inv_freq, conc), dtype)
    cache.append(k_rot, np.asarray(v, dtype=np.float64))
    out = sink_attention(q_rot, cache.K, cache.V, sinks, o, window, sm_scale)
    return out, q_rot, k_rot


def decode_step(cache, q, k, v, sinks, window, sm_scale, inv_freq, conc,
                dtype):
    """One token per sequence: q [B,1,n_q,d], k/v [B,1,n_kv,d]."""
    if q.shape[1] != 1:
        raise ValueError("decode takes exactly one token per step")
    return prefill_layer(cache, q, k, v, sinks, window, sm_scale, inv_freq,
                         conc, dtype)
