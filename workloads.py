"""Seeded synthetic inputs and workload shapes for the sink-GQA attention path.

This module holds none of the method's arithmetic: only the five workload
shapes, seeded random draws, and the rounding of those draws to the storage
dtype (bf16 round-to-nearest-even from float32).  It is the one module that
both the fp64 oracle checks and the HIP path consume, so that both see the
same host tensors.

Draw recipe: ``numpy.random.Generator(PCG64(SeedSequence([seed, cfg, layer,
tensor])))``, standard normal in float32, then rounded to bf16 when the
workload stores bf16.  Decode step ``s`` draws its new token's q, k, v from
tensor ids ``100 + 3*s + {0, 1, 2}``.  Sinks stay float32.

The shapes follow the pages: the gpt-oss attention block (64 query heads of
width 64, 8 KV heads, a 128-token band; "GQA Attention" study note, "How it
works") and GPT-OSS-Lite (8 query heads, 4 KV heads, head dim 96; GPT-OSS-Lite
visual guide, "Architecture Specifications").
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

# Tensor ids inside one (seed, cfg, layer) stream.
T_Q, T_K, T_V, T_SINK, T_PREFIX_K, T_PREFIX_V = 0, 1, 2, 3, 4, 5
T_DECODE_BASE = 100


@dataclass(frozen=True)
class Yarn:
    """YaRN / NTK-by-parts parameters (s = factor; s == 1 is plain RoPE)."""
    base: float = 150000.0
    factor: float = 32.0
    orig_ctx: int = 4096
    alpha: float = 1.0
    beta: float = 32.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    n_q: int
    n_kv: int
    d_h: int
    dtype: str                    # "bf16" or "f32"
    T: int                        # new query tokens of the prefill (0: none)
    windows: Tuple[int, ...]      # one entry per layer kind; 0 = full causal
    yarn: Yarn
    sm_scale: float
    prefix: int = 0               # rows already in the cache before the prefill
    decode_steps: int = 0
    capacity: int = 0             # cache rows (multiple of 32)
    seed: int = 0
    cfg_idx: int = 0

    @property
    def q_mult(self) -> int:
        return self.n_q // self.n_kv

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _cap(rows: int) -> int:
    return ((rows + 63) // 64) * 64


# The five workloads.  Window 0 means the full causal triangle.
TINY_F32 = Workload(
    name="tiny-f32 B1 T128 8/2 d64", B=1, n_q=8, n_kv=2, d_h=64, dtype="f32",
    T=128, windows=(0, 32), yarn=Yarn(base=10000.0, factor=1.0),
    sm_scale=1.0 / 8.0, capacity=128, cfg_idx=0)

LITE_PREFILL = Workload(
    name="gpt-oss-lite prefill B4 T4096 8/4 d96", B=4, n_q=8, n_kv=4, d_h=96,
    dtype="bf16", T=4096, windows=(128, 0), yarn=Yarn(),
    sm_scale=1.0 / np.sqrt(96.0), capacity=4096, cfg_idx=1)

GPTOSS_PREFILL = Workload(
    name="gpt-oss prefill B1 T8192 64/8 d64", B=1, n_q=64, n_kv=8, d_h=64,
    dtype="bf16", T=8192, windows=(128, 0), yarn=Yarn(), sm_scale=1.0 / 8.0,
    capacity=8192, cfg_idx=2)

LONG_DECODE = Workload(
    name="long decode B8 ctx131072 64/8 d64", B=8, n_q=64, n_kv=8, d_h=64,
    dtype="bf16", T=0, windows=(0, 128), yarn=Yarn(), sm_scale=1.0 / 8.0,
    prefix=131071, decode_steps=64, capacity=_cap(131071 + 64), cfg_idx=3)

HANDOVER = Workload(
    name="handover B1 65536+2048 64/8 d64", B=1, n_q=64, n_kv=8, d_h=64,
    dtype="bf16", T=2048, windows=(128, 0), yarn=Yarn(), sm_scale=1.0 / 8.0,
    prefix=65536, decode_steps=32, capacity=_cap(65536 + 2048 + 64),
    cfg_idx=4)

ALL = (TINY_F32, LITE_PREFILL, GPTOSS_PREFILL, LONG_DECODE, HANDOVER)


# --------------------------------------------------------------------------
# draws

def rng(seed: int, cfg: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, cfg, layer, tensor])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(shape, dtype: str, seed: int, cfg: int, layer: int,
           tensor: int, chunk_rows: int = 1 << 22) -> np.ndarray:
    """N(0,1) float32 draw of ``shape``; bf16-exact values when dtype=='bf16'.

    Large draws are produced in slabs along the first axis' flattened order
    so the float32 temporary stays bounded; the values do not depend on the
    slab size (one generator, consumed in order)."""
    g = rng(seed, cfg, layer, tensor)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    step = max(1, chunk_rows)
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)
        if dtype == "bf16":
            out[s:e] = bf16_round(out[s:e])
    return out.reshape(shape)


def sinks(w: Workload, layer: int) -> np.ndarray:
    g = rng(w.seed, w.cfg_idx, layer, T_SINK)
    return g.standard_normal(w.n_q, dtype=np.float32)


def prefill_inputs(w: Workload, layer: int) -> Dict[str, np.ndarray]:
    """q [B,T,n_q,d], k/v [B,T,n_kv,d] (pre-RoPE), sinks [n_q] and, when the
    workload has a prefix, the already-cached rows prefix_k/prefix_v
    [B,prefix,n_kv,d] (the K rows count as already rotated)."""
    out = {
        "q": normal((w.B, w.T, w.n_q, w.d_h), w.dtype, w.seed, w.cfg_idx, layer, T_Q),
        "k": normal((w.B, w.T, w.n_kv, w.d_h), w.dtype, w.seed, w.cfg_idx, layer, T_K),
        "v": normal((w.B, w.T, w.n_kv, w.d_h), w.dtype, w.seed, w.cfg_idx, layer, T_V),
        "sinks": sinks(w, layer),
    }
    if w.prefix:
        out.update(prefix_inputs(w, layer))
    return out


def prefix_inputs(w: Workload, layer: int) -> Dict[str, np.ndarray]:
    return {
        "prefix_k": normal((w.B, w.prefix, w.n_kv, w.d_h), w.dtype, w.seed,
                           w.cfg_idx, layer, T_PREFIX_K),
        "prefix_v": normal((w.B, w.prefix, w.n_kv, w.d_h), w.dtype, w.seed,
                           w.cfg_idx, layer, T_PREFIX_V),
    }


def decode_token(w: Workload, layer: int, step: int,
                 seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """The new token of decode step ``step``: q [B,1,n_q,d], k/v [B,1,n_kv,d]."""
    s = w.seed if seed is None else seed
    base = T_DECODE_BASE + 3 * step
    return {
        "q": normal((w.B, 1, w.n_q, w.d_h), w.dtype, s, w.cfg_idx, layer, base),
        "k": normal((w.B, 1, w.n_kv, w.d_h), w.dtype, s, w.cfg_idx, layer, base + 1),
        "v": normal((w.B, 1, w.n_kv, w.d_h), w.dtype, s, w.cfg_idx, layer, base + 2),
    }


# ---------------------------------------------------------------- sampling
# Rows of fp32 logits over the GPT-OSS-Lite vocabulary (128,000 tokens,
# GPT-OSS-Lite README model diagram) at the long-context decode batch (8).
SAMPLE_B, SAMPLE_V = 8, 128000
T_SAMPLE_LOGITS, T_SAMPLE_HISTORY, T_SAMPLE_U, T_SAMPLE_BIAS = 200, 201, 202, 203


def sampling_inputs(B: int, V: int, seed: int, scale: float = 2.0, history: int = 64,
                    bf16_logits: bool = False) -> Dict[str, np.ndarray]:
    """logits = scale * N(0, 1) fp32 [B, V] (bf16-rounded when asked, so that
    equal logits occur); history: `history` token ids per row drawn
    uniformly from [0, V) (int32); u: one uniform in [0, 1) per row
    (float32); bias: N(0, 1) fp32 [V]."""
    z = (rng(seed, 7, 0, T_SAMPLE_LOGITS).standard_normal((B, V), dtype=np.float32) * np.float32(scale))
    if bf16_logits:
        z = bf16_round(z)
    h = rng(seed, 7, 0, T_SAMPLE_HISTORY).integers(0, V, size=(B, history)).astype(np.int32)
    u = rng(seed, 7, 0, T_SAMPLE_U).random(B, dtype=np.float32)
    bias = rng(seed, 7, 0, T_SAMPLE_BIAS).standard_normal(V, dtype=np.float32)
    return {"logits": z.astype(np.float32), "history": h, "u": u, "bias": bias}
