"""Sliding-window ring cache for band layers -- oracle, test infrastructure.

What the pages fix:
  * "GPT-OSS-Lite" README, "Why these metrics matter": the windowed layers
    keep only the last 128 tokens in their cache while the full-attention
    layers keep the whole sequence; the KV-cache reduction this gives is the
    architecture's headline claim ("Results", KV-cache reduction table:
    about 1.94x at 4K tokens, because the windowed layers hold 128 rows
    whatever the length; "Headline benchmark": 2.00x).
  * "GPT-OSS-Lite" visual guide, KV-cache calculator: the count is of
    logical bf16 K/V entries, 12 layers, 4 KV heads, head_dim 96; ring
    duplication and temporaries are not counted.
  * "MoE-Xtend" README, ARCHITECTURE: with sliding-window layers a decode
    step's attention is O(W); ATTENTION STACK: sliding window on alternating
    layers (layer_idx % 2 == 0).

Reading (the pages name the ring only by what it stores; the plainest form
that fits): a band layer of width W keeps W rows per sequence.  The row of
global position p lives in slot p mod W, so appending p overwrites p - W,
the one key that has just left the band of the query at p (band of W keys
including the diagonal, as the attention oracle reads the pages).  After
positions [0, n) have been appended, slot s holds

    pos(s) = (n - 1) - ((n - 1 - s) mod W)   if that is >= 0, else nothing.

The band mask in ring coordinates, for a query at p: slot s is allowed iff
it holds a position and p - W < pos(s) <= p.  For the decode query
(p = n - 1) that is every slot that holds a row.

A prefill chunk at positions [o, o + T) needs keys down to o - W + 1 for its
first query but up to o + T - 1 for its last, more than W rows when T > 1,
so a chunk attends over the ring's live rows below o together with the
chunk's own rows, and only then are the chunk's rows written into the ring
(the last W of them survive).

Snapshot/restore on a ring: appends overwrite slots, so a ring is restored
by copying its W rows back (save/load), not by moving the offset.
"""
import itertools

import numpy as np

from .attention import attend_query

_ids = itertools.count(1)


def ring_slot(p: int, W: int) -> int:
    """Slot of global position p in a ring of W rows."""
    return p % W


def ring_positions(n: int, W: int) -> np.ndarray:
    """Position held by each of the W slots after positions [0, n) were
    appended in order; -1 where a slot holds nothing yet."""
    pos = np.full(W, -1, dtype=np.int64)
    for p in range(n):                     # replay the appends one by one
        pos[ring_slot(p, W)] = p
    return pos


def ring_positions_closed(n: int, W: int) -> np.ndarray:
    """The same as ring_positions, from the closed form
    pos(s) = (n-1) - ((n-1-s) mod W), negative meaning empty."""
    s = np.arange(W, dtype=np.int64)
    pos = (n - 1) - np.mod(n - 1 - s, W)
    return np.where(pos >= 0, pos, -1)


def ring_mask(p: int, n: int, W: int) -> np.ndarray:
    """Band mask in ring coordinates: bool [W], slot s allowed for a query at
    position p (p <= n - 1) of a ring holding positions [0, n)."""
    pos = ring_positions_closed(n, W)
    return (pos >= 0) & (pos > p - W) & (pos <= p)


def kv_entries(T: int, W: int, n_layers: int, ring: bool) -> int:
    """Cached rows per sequence and KV head, summed over the layers: full
    layers hold T rows; band layers (even layer index) hold min(T, W) with a
    ring, T without."""
    total = 0
    for layer in range(n_layers):
        band = layer % 2 == 0
        total += min(T, W) if (band and ring) else T
    return total


def kv_reduction(T: int, W: int, n_layers: int = 12) -> float:
    """KV entries of an all-full-cache model over those of the ring model."""
    return kv_entries(T, W, n_layers, False) / kv_entries(T, W, n_layers, True)


class OracleRingCache:
    """Ring of W rows per sequence for one band layer; rows stored as float64
    values of the storage dtype.  offset = positions appended so far."""

    def __init__(self, B: int, W: int, n_kv: int, d: int, fill: float = np.nan):
        self.B, self.W, self.n_kv, self.d = B, W, n_kv, d
        self.K = np.full((B, W, n_kv, d), fill, dtype=np.float64)
        self.V = np.full((B, W, n_kv, d), fill, dtype=np.float64)
        self.offset = 0
        self.cache_id = next(_ids)

    def append(self, k_rot: np.ndarray, v: np.ndarray) -> None:
        """k_rot, v [B, T_new, n_kv, d]: row t is position offset + t and goes
        to its slot; rows are written in order, so of two rows W apart the
        later one stays."""
        T_new = k_rot.shape[1]
        if k_rot.shape != (self.B, T_new, self.n_kv, self.d) or v.shape != k_rot.shape:
            raise ValueError("shape mismatch")
        for t in range(T_new):
            s = ring_slot(self.offset + t, self.W)
            self.K[:, s] = k_rot[:, t]
            self.V[:, s] = v[:, t]
        self.offset += T_new

    def live(self):
        """(positions [W], bool live [W]) of the slots."""
        pos = ring_positions_closed(self.offset, self.W)
        return pos, pos >= 0

    def save(self):
        return (self.cache_id, self.offset, self.K.copy(), self.V.copy())

    def load(self, saved) -> None:
        cache_id, off, K, V = saved
        if cache_id != self.cache_id:
            raise ValueError("saved state of another ring")
        self.offset = off
        self.K[...] = K
        self.V[...] = V


def _attend_rows(q_heads, K_rows, V_rows, sinks, sm_scale):
    """Sink attention of one token over the given rows, all allowed
    ([n, n_kv, d] each): the attention oracle's per-query form with a band
    that admits every row handed to it."""
    n = K_rows.shape[0]
    return attend_query(q_heads, K_rows, V_rows, sinks, n - 1, 0, sm_scale)


def ring_decode(ring: OracleRingCache, q_rot: np.ndarray, sinks: np.ndarray,
                sm_scale: float) -> np.ndarray:
    """Attention of the decode token (position p = offset - 1, its own row
    already appended) over the ring, in slot order with the ring mask.
    q_rot [B, 1, n_q, d]; returns fp64 [B, 1, n_q, d]."""
    p = ring.offset - 1
    if p < 0:
        raise ValueError("append the step's row first")
    m = ring_mask(p, ring.offset, ring.W)
    slots = np.nonzero(m)[0]
    B, _, n_q, d = q_rot.shape
    out = np.empty((B, 1, n_q, d), dtype=np.float64)
    for b in range(B):
        out[b, 0] = _attend_rows(q_rot[b, 0], ring.K[b, slots], ring.V[b, slots], sinks,
                                 sm_scale)
    return out


def ring_prefill(ring: OracleRingCache, q_rot: np.ndarray, k_rot: np.ndarray,
                 v: np.ndarray, sinks: np.ndarray, sm_scale: float) -> np.ndarray:
    """A chunk at positions [o, o + T), o = ring.offset: each query attends
    over the band among the ring's live rows (positions < o) and the chunk's
    rows; then the chunk is appended to the ring.  q_rot [B,T,n_q,d],
    k_rot / v [B,T,n_kv,d]; returns fp64 [B,T,n_q,d]."""
    o, W = ring.offset, ring.W
    B, T, n_q, d = q_rot.shape
    pos_r, live = ring.live()
    pos_all = np.concatenate([pos_r[live], o + np.arange(T)])
    out = np.empty((B, T, n_q, d), dtype=np.float64)
    for b in range(B):
        K_all = np.concatenate([ring.K[b, live], np.asarray(k_rot[b], np.float64)])
        V_all = np.concatenate([ring.V[b, live], np.asarray(v[b], np.float64)])
        for t in range(T):
            p = o + t
            sel = np.nonzero((pos_all > p - W) & (pos_all <= p))[0]
            out[b, t] = _attend_rows(q_rot[b, t], K_all[sel], V_all[sel], sinks, sm_scale)
    ring.append(k_rot, np.asarray(v, np.float64))
    return out
