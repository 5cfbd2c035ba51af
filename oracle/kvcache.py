"""Append-only KV cache with snapshot/restore -- oracle, test infrastructure.

"MoE-Xtend" README:
  * KV CACHE: per layer K, V are preallocated [B, T_cache, H_kv, d]; extend
    writes the new rows at [offset, offset + t) and then advances offset;
    snapshot()/restore() support "prefill once, decode many";
  * DESIGN CONTRACTS: append-only; decode adds exactly one row per layer per
    step and offset moves once per append;
  * KV CACHE, memory scaling: bytes ~ 2 * L * B * T * H_kv * d * dtype_bytes.

Snapshot reading (the pages give only the names): a snapshot records the
offset; restore rewinds the offset to it.  Rows below a snapshot's offset are
never rewritten by appends at or above that offset, so a restore is exact as
long as no append since the snapshot started below the snapshot's offset.
Such a later-invalidated snapshot is refused.  One offset is shared by all
sequences of the batch (the cache carries a single scalar offset).
"""
import itertools

import numpy as np


def kv_cache_bytes(L: int, B: int, T: int, H_kv: int, d: int,
                   dtype_bytes: int) -> int:
    """2 * L * B * T * H_kv * d * dtype_bytes (the factor 2 is K and V)."""
    return 2 * L * B * T * H_kv * d * dtype_bytes


class SnapshotError(RuntimeError):
    pass


_ids = itertools.count(1)


class OracleKVCache:
    """Host cache; rows are stored as float64 values of the storage dtype."""

    def __init__(self, B: int, capacity: int, n_kv: int, d: int,
                 fill: float = np.nan):
        self.B, self.capacity, self.n_kv, self.d = B, capacity, n_kv, d
        self.K = np.full((B, capacity, n_kv, d), fill, dtype=np.float64)
        self.V = np.full((B, capacity, n_kv, d), fill, dtype=np.float64)
        self.offset = 0
        self.cache_id = next(_ids)
        self.stamp = 0
        self._writes = []            # (stamp, first_row) of every append

    def append(self, k_rot: np.ndarray, v: np.ndarray) -> None:
        """k_rot, v [B, T_new, n_kv, d]; writes rows [offset, offset+T_new)."""
        T_new = k_rot.shape[1]
        if k_rot.shape != (self.B, T_new, self.n_kv, self.d) or v.shape != k_rot.shape:
            raise ValueError("shape mismatch")
        if self.offset + T_new > self.capacity:
            raise ValueError("capacity exceeded")
        o = self.offset
        self.K[:, o:o + T_new] = k_rot
        self.V[:, o:o + T_new] = v
        self.stamp += 1
        self._writes.append((self.stamp, o))
        self.offset = o + T_new

    def snapshot(self):
        return (self.cache_id, self.offset, self.stamp)

    def restore(self, snap) -> None:
        cache_id, off, stamp = snap
        if cache_id != self.cache_id:
            raise SnapshotError("snapshot of another cache")
        for s, first in self._writes:
            if s > stamp and first < off:
                raise SnapshotError("rows below the snapshot were rewritten")
        self.offset = off
