"""Shared plumbing of the GPU parity tests: host <-> device copies, the
library's layer step (RoPE, append, attend) and the oracle's counterpart."""
import numpy as np
import torch

import long_context_sparse_yarn_amd as sa
from oracle.attention import attend_query, sink_attention
from oracle.rounding import round_to
from oracle.yarn import rope_apply, yarn_concentration, yarn_inv_freq

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
TOL = {"bf16": 2e-2, "f32": 1e-5}


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host float32 values (bf16-exact for bf16) -> device tensor, exact."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(TORCH_DT[dtype])


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def lib_yarn(d, y) -> "sa.Yarn":
    return sa.Yarn(d, y.base, y.factor, y.orig_ctx, y.alpha, y.beta)


def oracle_tables(d, y):
    return (yarn_inv_freq(d, y.base, y.factor, y.orig_ctx, y.alpha, y.beta),
            yarn_concentration(y.factor))


def oracle_rot(x, offset, d, y, dtype):
    inv, c = oracle_tables(d, y)
    return round_to(rope_apply(np.asarray(x, np.float64), offset, inv, c), dtype)


def gpu_prefill_layer(cache, q, k, v, sinks_t, window, sm_scale, y, dtype):
    """Library path for one chunk: rotate Q/K at the cache offset, append,
    attend.  q/k/v are host arrays; returns (out, q_rot, k_rot) device tensors."""
    d = q.shape[-1]
    o = cache.offset
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    ly = lib_yarn(d, y)
    sa.yarn_rope_apply(qd, o, ly)
    sa.yarn_rope_apply(kd, o, ly)
    cache.append(kd, vd)
    out = sa.sinkattn_prefill(qd, cache, sinks_t, window, sm_scale, o)
    return out, qd, kd


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
