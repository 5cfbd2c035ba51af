"""Pins for the oracle's KV cache ("MoE-Xtend" README, KV CACHE)."""
import json
import os

import numpy as np
import pytest

from oracle.kvcache import OracleKVCache, SnapshotError, kv_cache_bytes
from oracle.layer import decode_step, prefill_layer
from oracle.yarn import yarn_concentration, yarn_inv_freq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_bytes_printed_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_example.json")))
    n = kv_cache_bytes(g["L"], g["B"], g["T"], g["H_kv"], g["d"], g["dtype_bytes"])
    assert n / 2 ** 30 == g["printed_gib"]          # 6.0 GiB exactly
    assert n == 6442450944


def test_kv_bytes_counts_k_and_v():
    # one layer, one row, one head: K and V rows of d elements each
    assert kv_cache_bytes(1, 1, 1, 1, 64, 2) == 2 * 64 * 2
    # linear in every factor
    assert kv_cache_bytes(2, 3, 5, 7, 11, 4) == 2 * 2 * 3 * 5 * 7 * 11 * 4


def test_append_places_rows_and_advances():
    c = OracleKVCache(2, 10, 3, 4)
    k = np.arange(2 * 3 * 3 * 4, dtype=float).reshape(2, 3, 3, 4)
    c.append(k, -k)
    assert c.offset == 3
    assert np.array_equal(c.K[:, :3], k) and np.array_equal(c.V[:, :3], -k)
    assert np.all(np.isnan(c.K[:, 3:]))
    c.append(k[:, :1], k[:, :1])
    assert c.offset == 4 and np.array_equal(c.K[:, 3], k[:, 0])
    with pytest.raises(ValueError):
        c.append(np.zeros((2, 7, 3, 4)), np.zeros((2, 7, 3, 4)))


def test_snapshot_restore_prefill_once_decode_many():
    B, n_q, n_kv, d = 1, 4, 2, 8
    inv = yarn_inv_freq(d, 150000.0, 32.0, 4096, 1.0, 32.0)
    cc = yarn_concentration(32.0)
    rng = np.random.default_rng(0)
    s = rng.standard_normal(n_q)
    c = OracleKVCache(B, 64, n_kv, d)
    prefill_layer(c, rng.standard_normal((B, 20, n_q, d)), rng.standard_normal((B, 20, n_kv, d)),
                  rng.standard_normal((B, 20, n_kv, d)), s, 0, 0.3, inv, cc, "bf16")
    snap = c.snapshot()

    def sweep(seed):
        r = np.random.default_rng(seed)
        outs = []
        for _ in range(5):
            o, _, _ = decode_step(c, r.standard_normal((B, 1, n_q, d)),
                                  r.standard_normal((B, 1, n_kv, d)),
                                  r.standard_normal((B, 1, n_kv, d)), s, 0, 0.3, inv, cc, "bf16")
            outs.append(o)
        return np.concatenate(outs, 1)

    a1 = sweep(1)
    c.restore(snap)
    assert c.offset == 20
    b = sweep(2)
    c.restore(snap)
    a2 = sweep(1)
    assert np.array_equal(a1, a2)
    assert not np.allclose(a1, b)


def test_stale_and_foreign_snapshots_refused():
    c = OracleKVCache(1, 32, 1, 2)
    one = np.ones((1, 1, 1, 2))
    for _ in range(5):
        c.append(one, one)
    early = c.snapshot()                # offset 5
    for _ in range(5):
        c.append(one, one)
    late = c.snapshot()                 # offset 10
    c.restore(early)
    c.append(one, one)                  # rewrites row 5 < 10
    with pytest.raises(SnapshotError):
        c.restore(late)
    c.restore(early)                    # row 5 is not below early's offset
    assert c.offset == 5
    other = OracleKVCache(1, 32, 1, 2)
    with pytest.raises(SnapshotError):
        other.restore(early)
