"""Pins for the oracle's fused qkv projection (oracle/qkv.py): the printed
widths, a written-out triple loop, the [Q | K | V] head-major split read back
through one-hot weights, the bias, and the single rounding of a bf16 layer."""
import json
import os

import numpy as np
import pytest

from oracle.layer import prefill_layer
from oracle.kvcache import OracleKVCache
from oracle.qkv import qkv_project, qkv_split, qkv_width
from oracle.rounding import round_to
from oracle.yarn import yarn_concentration, yarn_inv_freq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return round_to(np.asarray(a, np.float64), "bf16")


def test_widths_printed_on_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "gpt_oss_attention_shapes.json")))
    assert qkv_width(g["n_q"], g["n_kv"], g["d_h"]) == g["d_qkv"] == 5120
    lite = json.load(open(os.path.join(GOLDEN, "gpt_oss_lite_shapes.json")))
    assert qkv_width(lite["n_q"], lite["n_kv"], lite["d_h"]) == 96 * 16


def test_projection_equals_a_written_out_loop():
    rng = np.random.default_rng(0)
    T, dm, n_q, n_kv, d = 3, 5, 2, 1, 2
    N = qkv_width(n_q, n_kv, d)
    x, W, b = _bf16(rng.standard_normal((T, dm))), _bf16(rng.standard_normal((N, dm))), \
        _bf16(rng.standard_normal(N))
    want = np.empty((T, N))
    for t in range(T):
        for n in range(N):
            acc = b[n]
            for j in range(dm):
                acc += x[t, j] * W[n, j]
            want[t, n] = acc
    assert np.array_equal(qkv_project(x, W, b), round_to(want, "bf16"))


def test_bias_alone_and_zero_weights():
    rng = np.random.default_rng(1)
    b = _bf16(rng.standard_normal(24))
    out = qkv_project(rng.standard_normal((4, 8)), np.zeros((24, 8)), b)
    assert np.array_equal(out, np.broadcast_to(b, (4, 24)))


@pytest.mark.parametrize("n_q,n_kv,d", [(4, 2, 8), (3, 1, 4), (64, 8, 64)])
def test_split_is_q_k_v_head_major(n_q, n_kv, d):
    """A one-hot weight row n copies input column j into output column n;
    the split must put it at (part, head, coordinate) of the layout."""
    rng = np.random.default_rng(n_q)
    N = qkv_width(n_q, n_kv, d)
    dm = 7
    x = _bf16(rng.standard_normal((2, dm)))
    for n in rng.choice(N, size=min(N, 20), replace=False):
        j = int(rng.integers(dm))
        W = np.zeros((N, dm))
        W[n, j] = 1.0
        q, k, v = qkv_split(qkv_project(x, W, np.zeros(N)), n_q, n_kv, d)
        parts = [("q", q, n_q), ("k", k, n_kv), ("v", v, n_kv)]
        start, hit = 0, None
        for name, arr, heads in parts:
            if n < start + heads * d:
                hit = (name, arr, (n - start) // d, (n - start) % d)
                break
            start += heads * d
        name, arr, h, e = hit
        assert np.array_equal(arr[:, h, e], x[:, j]), (n, name, h, e)
        assert np.count_nonzero(q) + np.count_nonzero(k) + np.count_nonzero(v) == \
            np.count_nonzero(x[:, j])


def test_rounded_once_not_per_term():
    # bf16 ulp at 1 is 2^-7; 3*2^-10 is 0.375 ulp.  Rounding each partial sum
    # to bf16 would keep 1 twice; the exact 1 + 0.75 ulp rounds to 1 + 2^-7
    t = 3.0 * 2.0 ** -10
    x = np.array([[1.0, t, t]])
    W = np.array([[1.0, 1.0, 1.0]])
    assert qkv_project(x, W, np.zeros(1))[0, 0] == 1.0 + 2.0 ** -7
    # the bias joins before the one rounding
    assert qkv_project(x[:, :2], W[:, :2], np.array([t]))[0, 0] == 1.0 + 2.0 ** -7
    # and one term alone stays below the midpoint
    assert qkv_project(x[:, :2], W[:, :2], np.zeros(1))[0, 0] == 1.0


def test_layer_from_hidden_states_composes():
    """Projection, split, RoPE at the offset and append: the layer oracle on
    the split parts, unchanged."""
    rng = np.random.default_rng(3)
    B, T, dm, n_q, n_kv, d = 2, 6, 16, 4, 2, 8
    N = qkv_width(n_q, n_kv, d)
    x, W, b = _bf16(rng.standard_normal((B, T, dm))), _bf16(0.3 * rng.standard_normal((N, dm))), \
        _bf16(rng.standard_normal(N))
    qkv = qkv_project(x, W, b)
    assert qkv.shape == (B, T, N)
    q, k, v = qkv_split(qkv, n_q, n_kv, d)
    inv, c = yarn_inv_freq(d, 150000.0, 32.0, 4096, 1.0, 32.0), yarn_concentration(32.0)
    cache = OracleKVCache(B, 32, n_kv, d)
    cache.append(_bf16(rng.standard_normal((B, 5, n_kv, d))), _bf16(rng.standard_normal((B, 5, n_kv, d))))
    out, q_rot, k_rot = prefill_layer(cache, q, k, v, rng.standard_normal(n_q), 0, 0.35, inv, c, "bf16")
    assert cache.offset == 5 + T
    assert np.array_equal(cache.V[:, 5:5 + T], v)
    assert np.array_equal(cache.K[:, 5:5 + T], k_rot)
    assert np.all(np.isfinite(out))
