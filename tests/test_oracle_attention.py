"""Pins for the oracle's sink-GQA attention.

The oracle is held against: its own dense mask-matrix form (brute force on
tiny shapes); PyTorch's CPU fp64 scaled_dot_product_attention (a library
routine) with an explicit boolean mask, with the sink written as one extra
key column; closed forms of the leaky normalisation; exact mask-edge probes;
and the decode == prefill and chunked-prefill invariants of the pages.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle.kvcache import OracleKVCache
from oracle.layer import decode_step, prefill_layer
from oracle.yarn import yarn_concentration, yarn_inv_freq


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(B, T, n_q, n_kv, d, n_ctx, seed, sink_inf=False):
    q = _rand((B, T, n_q, d), seed)
    K = _rand((B, n_ctx, n_kv, d), seed + 1)
    V = _rand((B, n_ctx, n_kv, d), seed + 2)
    s = np.full(n_q, -np.inf) if sink_inf else _rand(n_q, seed + 3)
    return q, K, V, s


SHAPES = [
    # B, T, n_q, n_kv, d, offset, window
    (1, 16, 4, 4, 8, 0, 0),
    (2, 33, 8, 2, 8, 5, 7),
    (1, 40, 6, 3, 64, 0, 16),
    (1, 24, 8, 1, 96, 17, 0),
    (2, 64, 4, 2, 64, 0, 1),
    (1, 20, 16, 2, 8, 30, 128),
]


@pytest.mark.parametrize("B,T,n_q,n_kv,d,off,W", SHAPES)
@pytest.mark.parametrize("sink_inf", [False, True])
def test_per_query_form_equals_dense_form(B, T, n_q, n_kv, d, off, W, sink_inf):
    n_ctx = off + T + 3                      # written rows past the last query
    q, K, V, s = _case(B, T, n_q, n_kv, d, n_ctx, 10 + d, sink_inf)
    a = A.sink_attention(q, K, V, s, off, W, 0.3)
    b = A.sink_attention_dense(q, K, V, s, off, W, 0.3)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def _bool_mask(T, n_ctx, off, W):
    qi = torch.arange(T)[:, None] + off
    kj = torch.arange(n_ctx)[None, :]
    m = kj <= qi
    if W > 0:
        m &= kj > qi - W
    return m


@pytest.mark.parametrize("B,T,n_q,n_kv,d,off,W", SHAPES)
def test_no_sink_equals_torch_sdpa(B, T, n_q, n_kv, d, off, W):
    n_ctx = off + T
    q, K, V, s = _case(B, T, n_q, n_kv, d, n_ctx, 20 + T, sink_inf=True)
    got = A.sink_attention(q, K, V, s, off, W, 0.25)
    qm = n_q // n_kv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)                    # B,H,T,d
    tk = torch.from_numpy(K).repeat_interleave(qm, dim=2).permute(0, 2, 1, 3)
    tv = torch.from_numpy(V).repeat_interleave(qm, dim=2).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=_bool_mask(T, n_ctx, off, W),
                                         scale=0.25).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("B,T,n_q,n_kv,d,off,W", SHAPES)
def test_sink_is_an_extra_dropped_column(B, T, n_q, n_kv, d, off, W):
    # The sink column equals one extra key with score sigma_h and value 0.
    n_ctx = off + T
    q, K, V, s = _case(B, T, n_q, n_kv, d, n_ctx, 30 + T)
    s = s * 3.0
    got = A.sink_attention(q, K, V, s, off, W, 0.25)
    qm = n_q // n_kv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(K).repeat_interleave(qm, dim=2).permute(0, 2, 1, 3)
    tv = torch.from_numpy(V).repeat_interleave(qm, dim=2).permute(0, 2, 1, 3)
    tk = torch.cat([tk, torch.zeros(B, n_q, 1, d, dtype=tk.dtype)], 2)
    tv = torch.cat([tv, torch.zeros(B, n_q, 1, d, dtype=tv.dtype)], 2)
    add = torch.where(_bool_mask(T, n_ctx, off, W), 0.0, -torch.inf).to(torch.float64)
    add = add[None, None].expand(B, n_q, T, n_ctx)
    sink_col = torch.from_numpy(s)[None, :, None, None].expand(B, n_q, T, 1)
    mask = torch.cat([add, sink_col], -1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                         scale=0.25).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


def test_wide_band_equals_full_causal():
    q, K, V, s = _case(2, 30, 8, 2, 8, 50, 40)
    full = A.sink_attention(q, K, V, s, 20, 0, 0.5)
    for W in (50, 51, 1000):
        assert np.array_equal(A.sink_attention(q, K, V, s, 20, W, 0.5), full)


def test_gqa_equals_mha_with_repeated_kv():
    q, K, V, s = _case(1, 12, 8, 2, 16, 12, 50)
    g = A.sink_attention(q, K, V, s, 0, 5, 0.2)
    m = A.sink_attention(q, np.repeat(K, 4, axis=2), np.repeat(V, 4, axis=2), s, 0, 5, 0.2)
    np.testing.assert_allclose(g, m, atol=1e-14, rtol=0)
    # and head h really uses KV head h // q_mult: permuting KV heads moves outputs
    Kp, Vp = K[:, :, ::-1], V[:, :, ::-1]
    sp = np.concatenate([s[4:], s[:4]])
    qp = np.concatenate([q[:, :, 4:], q[:, :, :4]], axis=2)
    gp = A.sink_attention(qp, Kp, Vp, sp, 0, 5, 0.2)
    np.testing.assert_allclose(gp, np.concatenate([g[:, :, 4:], g[:, :, :4]], 2), atol=1e-14)


def test_leaky_normalisation_closed_form():
    # V == 1: out = sum e^l / (sum e^l + e^sigma) in every coordinate.
    q, K, V, s = _case(1, 9, 4, 2, 8, 9, 60)
    V = np.ones_like(V)
    out = A.sink_attention(q, K, V, s, 0, 0, 0.7)
    for t in range(9):
        for h in range(4):
            l = 0.7 * K[0, :t + 1, h // 2] @ q[0, t, h]
            ref = np.exp(l).sum() / (np.exp(l).sum() + np.exp(s[h]))
            np.testing.assert_allclose(out[0, t, h], ref, rtol=1e-13)


@pytest.mark.parametrize("W", [0, 1, 5, 128])
def test_mask_size_from_uniform_weights(W):
    # K == 0 makes every allowed logit 0; with V == 1 the output is
    # |A| / (|A| + e^sigma), so |A(p)| can be read back exactly.
    T, off = 40, 150
    q = _rand((1, T, 2, 8), 70)
    K = np.zeros((1, off + T, 1, 8))
    V = np.ones((1, off + T, 1, 8))
    s = np.array([0.3, -1.2])
    out = A.sink_attention(q, K, V, s, off, W, 1.0)
    for t in range(T):
        p = off + t
        for h in range(2):
            y = out[0, t, h, 0]
            n = y * np.exp(s[h]) / (1 - y)
            want = min(W, p + 1) if W > 0 else p + 1
            assert round(n) == want and abs(n - want) < 1e-8


def _probe(off, T, W, t, j):
    """Key j gets a +30 logit (after scaling) and a one-hot value."""
    d, n_ctx = 8, off + T
    q = np.zeros((1, T, 1, d))
    q[0, :, 0, 0] = 1.0
    K = np.zeros((1, n_ctx, 1, d))
    K[0, j, 0, 0] = 30.0
    V = np.zeros((1, n_ctx, 1, d))
    V[0, j, 0, 1] = 1.0
    out = A.sink_attention(q, K, V, np.array([-np.inf]), off, W, 1.0)
    return out[0, t, 0, 1]


@pytest.mark.parametrize("off,T", [(0, 300), (65536, 40), (7, 200)])
@pytest.mark.parametrize("W", [0, 128])
def test_mask_edges(off, T, W):
    for t in (0, 1, T // 2, T - 2):
        p = off + t
        assert _probe(off, T, W, t, p) > 0.99                  # diagonal allowed
        if p + 1 < off + T:
            assert _probe(off, T, W, t, p + 1) == 0.0          # future row masked
        if W > 0:
            if p - W + 1 >= 0:
                assert _probe(off, T, W, t, p - W + 1) > 0.99  # band edge allowed
            if p - W >= 0:
                assert _probe(off, T, W, t, p - W) == 0.0      # just outside


def _layer_inputs(B, T, n_q, n_kv, d, seed):
    return (_rand((B, T, n_q, d), seed), _rand((B, T, n_kv, d), seed + 1),
            _rand((B, T, n_kv, d), seed + 2), _rand(n_q, seed + 3))


@pytest.mark.parametrize("W", [0, 6])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_equal_one_prefill(W, dtype):
    B, T, n_q, n_kv, d = 2, 14, 4, 2, 8
    inv = yarn_inv_freq(d, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn_concentration(32.0)
    q, k, v, s = _layer_inputs(B, T, n_q, n_kv, d, 80)
    c1 = OracleKVCache(B, 32, n_kv, d)
    out1, _, _ = prefill_layer(c1, q, k, v, s, W, 0.35, inv, c, dtype)
    c2 = OracleKVCache(B, 32, n_kv, d)
    outs = []
    for t in range(T):
        o, _, _ = decode_step(c2, q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1],
                              s, W, 0.35, inv, c, dtype)
        outs.append(o)
        assert c2.offset == t + 1                      # exactly one row per step
    np.testing.assert_allclose(np.concatenate(outs, 1), out1, atol=1e-12, rtol=0)
    assert np.array_equal(c1.K[:, :T], c2.K[:, :T])
    assert np.array_equal(c1.V[:, :T], c2.V[:, :T])


@pytest.mark.parametrize("W", [0, 5])
def test_chunked_prefill_handover(W):
    # A prefill of T1 then a chunk of T2 at offset T1 equals one prefill of
    # T1+T2: the diagonal does not move at the handover.
    B, T1, T2, n_q, n_kv, d = 1, 11, 9, 4, 1, 8
    inv = yarn_inv_freq(d, 150000.0, 32.0, 4096, 1.0, 32.0)
    c = yarn_concentration(32.0)
    q, k, v, s = _layer_inputs(B, T1 + T2, n_q, n_kv, d, 90)
    whole = OracleKVCache(B, 64, n_kv, d)
    ref, _, _ = prefill_layer(whole, q, k, v, s, W, 0.3, inv, c, "f32")
    parts = OracleKVCache(B, 64, n_kv, d)
    a, _, _ = prefill_layer(parts, q[:, :T1], k[:, :T1], v[:, :T1], s, W, 0.3, inv, c, "f32")
    b, _, _ = prefill_layer(parts, q[:, T1:], k[:, T1:], v[:, T1:], s, W, 0.3, inv, c, "f32")
    np.testing.assert_allclose(np.concatenate([a, b], 1), ref, atol=1e-12, rtol=0)


def test_rows_past_the_query_are_never_read():
    # NaN in every cache row past the query position leaves outputs finite.
    q, K, V, s = _case(1, 10, 4, 2, 8, 30, 100)
    K[:, 10:] = np.nan
    V[:, 10:] = np.nan
    out = A.sink_attention(q, K, V, s, 0, 0, 0.5)
    assert np.all(np.isfinite(out))
