"""Fused qkv projection of one attention layer, feeding RoPE and the cache --
oracle, test infrastructure.

"GQA Attention" study note on gpt-oss, How it works: after RMSNorm the
residual stream x [T, d_model] goes through one fused linear layer "qkv" of
output width d_qkv = d_h (n_q + 2 n_kv) (5120 for gpt-oss: d_model 2880,
64 query heads and 8 KV heads of width 64); the result is split into Q
[T, n_q, d_h] and K, V [T, n_kv, d_h]; rotary embeddings run on Q and K only.
Both linear layers of the block are bf16 layers with a bias (the note calls
the biases an official-code detail).  "GPT-OSS-Lite" visual guide,
Architecture Specifications: d_model 768, 8 query heads, 4 KV heads,
d_head 96.

Readings (the note gives the width and the split, not the column order):
  * the fused width is laid out [Q | K | V], each part head-major
    (column h*d_h + e of a part is coordinate e of head h), the order in
    which the note lists the split;
  * the weight is stored as a linear layer's [d_qkv, d_model] matrix,
    qkv = x W^T + b;
  * a bf16 linear layer returns its product rounded once to bf16: the
    oracle forms x W^T + b exactly (fp64 on bf16 inputs; products of two
    bf16 values are exact in fp64 and the sums of up to a few thousand of
    them carry an error far below one bf16 ulp) and rounds to bf16 once.
Then Q and K are rotated at their global positions and K, V appended, as in
oracle/layer.py.
"""
import numpy as np

from .rounding import round_to


def qkv_width(n_q: int, n_kv: int, d: int) -> int:
    """d_qkv = d_h (n_q + 2 n_kv)."""
    return d * (n_q + 2 * n_kv)


def qkv_project(x: np.ndarray, W: np.ndarray, bias: np.ndarray,
                dtype: str = "bf16") -> np.ndarray:
    """x [..., d_model], W [d_qkv, d_model], bias [d_qkv] (values of the
    storage dtype) -> x W^T + b rounded once to dtype, as float64."""
    y = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T + np.asarray(bias, np.float64)
    return round_to(y, dtype)


def qkv_split(qkv: np.ndarray, n_q: int, n_kv: int, d: int):
    """[..., d_qkv] -> Q [..., n_q, d], K [..., n_kv, d], V [..., n_kv, d]."""
    lead = qkv.shape[:-1]
    if qkv.shape[-1] != qkv_width(n_q, n_kv, d):
        raise ValueError("width is not d (n_q + 2 n_kv)")
    q = qkv[..., :n_q * d].reshape(*lead, n_q, d)
    k = qkv[..., n_q * d:(n_q + n_kv) * d].reshape(*lead, n_kv, d)
    v = qkv[..., (n_q + n_kv) * d:].reshape(*lead, n_kv, d)
    return q, k, v
