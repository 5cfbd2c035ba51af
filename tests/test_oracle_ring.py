"""Pins for the oracle's sliding-window ring cache (oracle/ring.py).

The ring is held against things other than itself: the KV reductions the
GPT-OSS-Lite README prints, the closed form 2T/(T+W) of the alternating
layout, a replay of the appends against the closed-form slot positions, the
plain band mask of the attention oracle (bit-equal sets of allowed
positions), and the full-cache band attention of the oracle's linear cache.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.ring as ring_mod
from oracle.attention import allowed_range
from oracle.kvcache import OracleKVCache, kv_cache_bytes
from oracle.layer import decode_step, prefill_layer
from oracle.ring import (OracleRingCache, kv_entries, kv_reduction, ring_decode, ring_mask,
                         ring_positions, ring_positions_closed, ring_prefill)
from oracle.rounding import round_to
from oracle.yarn import rope_apply, yarn_concentration, yarn_inv_freq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_reduction_matches_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "kv_ring_reduction.json")))
    for row in g["printed"]:
        r = kv_reduction(row["T"], g["window"], g["n_layers"])
        assert round(r, row["digits"]) == row["reduction"], row
    lo, hi = g["printed_range"]
    for T in (4096, 8192, 32768, 65536, 131072):
        assert lo - 0.005 <= kv_reduction(T, g["window"], g["n_layers"]) <= hi


def test_reduction_closed_form():
    # half the layers full (T rows), half banded (W rows): 2T / (T + W)
    for T, W in ((4096, 128), (131072, 128), (1000, 32), (129, 128)):
        full = kv_entries(T, W, 12, ring=False)
        ring = kv_entries(T, W, 12, ring=True)
        assert Fraction(full, ring) == Fraction(2 * T, T + W)
    assert round(kv_reduction(4096, 128), 4) == 1.9394
    assert round(kv_reduction(131072, 128), 4) == 1.9980
    # shorter than the window: the ring holds everything, no reduction
    assert kv_reduction(100, 128) == 1.0
    # an odd layer count: 7 full + ... (layers 0, 2, 4, 6 banded)
    assert kv_entries(1000, 10, 7, ring=True) == 3 * 1000 + 4 * 10


def test_ring_bytes_at_128k_gpt_oss_lite():
    # 12 layers x 4 KV heads x 96, bf16, batch 1, 131072 tokens
    full = kv_cache_bytes(12, 1, 131072, 4, 96, 2)
    assert full / 2 ** 30 == 2.25
    ring = 2 * 1 * 4 * 96 * 2 * kv_entries(131072, 128, 12, ring=True)
    assert ring == kv_cache_bytes(6, 1, 131072, 4, 96, 2) + kv_cache_bytes(6, 1, 128, 4, 96, 2)
    assert round(ring / 2 ** 30, 3) == 1.126


@pytest.mark.parametrize("W", [1, 4, 5, 32, 128])
def test_slot_replay_equals_closed_form(W):
    for n in list(range(0, 3 * W + 6)) + [10 * W + 7]:
        assert np.array_equal(ring_positions(n, W), ring_positions_closed(n, W)), (n, W)


def test_planted_slot_mistake_is_caught(monkeypatch):
    # a ring that shifts every row by one slot no longer matches the closed form
    monkeypatch.setattr(ring_mod, "ring_slot", lambda p, W: (p + 1) % W)
    assert not np.array_equal(ring_mod.ring_positions(40, 32), ring_positions_closed(40, 32))


@pytest.mark.parametrize("W", [4, 5, 32, 128])
def test_ring_mask_bit_equals_band_mask(W):
    for n in list(range(1, 3 * W + 6)) + [7 * W + 3]:
        pos = ring_positions_closed(n, W)
        p = n - 1                                   # the decode query
        got = sorted(pos[ring_mask(p, n, W)].tolist())
        lo, hi = allowed_range(p, W)
        assert got == list(range(lo, hi)), (n, W)
        # earlier queries: the ring still holds their band above n - W
        for p in range(max(0, n - W), n):
            got = sorted(pos[ring_mask(p, n, W)].tolist())
            lo, hi = allowed_range(p, W)
            assert got == list(range(max(lo, n - W), hi)), (n, W, p)


def _setup(seed, d=8, n_q=4, n_kv=2):
    inv = yarn_inv_freq(d, 150000.0, 32.0, 4096, 1.0, 32.0)
    cc = yarn_concentration(32.0)
    rng = np.random.default_rng(seed)
    return inv, cc, rng, rng.standard_normal(n_q)


def _draw(rng, B, T, n_q, n_kv, d):
    return (rng.standard_normal((B, T, n_q, d)), rng.standard_normal((B, T, n_kv, d)),
            rng.standard_normal((B, T, n_kv, d)))


@pytest.mark.parametrize("W,chunks", [(8, [5, 3, 20, 1, 8]), (32, [40, 7, 64, 1]),
                                      (16, [16, 16, 3])])
def test_ring_prefill_and_decode_equal_full_cache_band(W, chunks):
    B, n_q, n_kv, d = 2, 4, 2, 8
    inv, cc, rng, sinks = _setup(W)
    sm = 0.35
    lin = OracleKVCache(B, sum(chunks) + 4 * W, n_kv, d)
    ring = OracleRingCache(B, W, n_kv, d)
    for T in chunks:                                # chunked prefill
        q, k, v = _draw(rng, B, T, n_q, n_kv, d)
        ref, q_rot, k_rot = prefill_layer(lin, q, k, v, sinks, W, sm, inv, cc, "bf16")
        got = ring_prefill(ring, q_rot, k_rot, v, sinks, sm)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    for _ in range(3 * W + 2):                      # decode wraps the ring several times
        q, k, v = _draw(rng, B, 1, n_q, n_kv, d)
        ref, q_rot, k_rot = decode_step(lin, q, k, v, sinks, W, sm, inv, cc, "bf16")
        ring.append(k_rot, v)
        got = ring_decode(ring, q_rot, sinks, sm)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert ring.offset == lin.offset
    # the ring holds exactly the last W rows of the linear cache, by slot
    n = lin.offset
    for p in range(n - W, n):
        assert np.array_equal(ring.K[:, p % W], lin.K[:, p])
        assert np.array_equal(ring.V[:, p % W], lin.V[:, p])


def test_ring_decode_before_the_ring_fills():
    B, n_q, n_kv, d, W = 1, 2, 1, 8, 32
    inv, cc, rng, sinks = _setup(3, d, n_q, n_kv)
    lin = OracleKVCache(B, 64, n_kv, d)
    ring = OracleRingCache(B, W, n_kv, d)          # NaN fill: empty slots must not be read
    for _ in range(W + 3):
        q, k, v = _draw(rng, B, 1, n_q, n_kv, d)
        ref, q_rot, k_rot = decode_step(lin, q, k, v, sinks, W, 0.5, inv, cc, "f32")
        ring.append(k_rot, v)
        got = ring_decode(ring, q_rot, sinks, 0.5)
        assert np.all(np.isfinite(got))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_ring_append_longer_than_window_keeps_last_rows():
    ring = OracleRingCache(1, 4, 1, 1)
    rows = np.arange(11, dtype=float).reshape(1, 11, 1, 1)
    ring.append(rows, -rows)
    assert ring.offset == 11
    # positions 7..10 survive, at slots 3, 0, 1, 2
    assert ring.K[0, :, 0, 0].tolist() == [8.0, 9.0, 10.0, 7.0]
    assert ring.V[0, :, 0, 0].tolist() == [-8.0, -9.0, -10.0, -7.0]


def test_save_load_prefill_once_decode_many():
    B, n_q, n_kv, d, W = 1, 4, 2, 8, 8
    inv, cc, rng, sinks = _setup(5)
    ring = OracleRingCache(B, W, n_kv, d)
    q, k, v = _draw(rng, B, 13, n_q, n_kv, d)
    q_rot = round_to(rope_apply(q, 0, inv, cc), "bf16")
    k_rot = round_to(rope_apply(k, 0, inv, cc), "bf16")
    ring_prefill(ring, q_rot, k_rot, v, sinks, 0.3)
    saved = ring.save()

    def sweep(seed):
        r = np.random.default_rng(seed)
        outs = []
        for _ in range(2 * W + 3):                 # overwrites every slot twice
            qq, kk, vv = _draw(r, B, 1, n_q, n_kv, d)
            p = ring.offset
            ring.append(round_to(rope_apply(kk, p, inv, cc), "bf16"), vv)
            outs.append(ring_decode(ring, round_to(rope_apply(qq, p, inv, cc), "bf16"),
                                    sinks, 0.3))
        return np.concatenate(outs, 1)

    a1 = sweep(1)
    ring.load(saved)
    assert ring.offset == 13
    b = sweep(2)
    ring.load(saved)
    a2 = sweep(1)
    assert np.array_equal(a1, a2)
    assert not np.allclose(a1, b)
    other = OracleRingCache(B, W, n_kv, d)
    with pytest.raises(ValueError):
        other.load(saved)
