"""Pins for the oracle's MoE layer (oracle/moe.py): brute-force top-k with the
stated tie-break, the softmax over the selected logits only, a dispatch that
lists every (token, slot) once in token order, SiLU's closed form, the
SwiGLU expert written out, and layer-level cases whose answer is known
(identical experts, all-equal logits, constant experts)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.moe import (dispatch, moe_layer, router_logits, silu, softmax_selected,
                        swiglu_expert, topk_stable)
from oracle.rounding import round_to

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return round_to(np.asarray(a, np.float64), "bf16")


def test_topk_brute_force_and_ties():
    rng = np.random.default_rng(0)
    # few distinct values: many ties
    S = rng.integers(-2, 3, size=(200, 6)).astype(np.float64)
    for k in (1, 2, 3, 6):
        I = topk_stable(S, k)
        for t in range(S.shape[0]):
            # every k-subset ordered by (-value, index); the chosen one is the first
            best = min(itertools.permutations(range(6), k),
                       key=lambda p: [(-S[t, e], e) for e in p])
            assert tuple(I[t]) == best
    S = np.zeros((1, 8))
    assert topk_stable(S, 2).tolist() == [[0, 1]]          # all equal: lowest ids
    S = np.array([[1.0, 3.0, 3.0, 2.0]])
    assert topk_stable(S, 2).tolist() == [[1, 2]]
    assert topk_stable(S, 3).tolist() == [[1, 2, 3]]


def test_softmax_over_selected_only():
    S = np.array([[0.0, 1.0, 5.0, 2.0]])
    I = np.array([[2, 3]])
    w = softmax_selected(S, I)
    assert np.allclose(w, [[np.exp(3.0) / (np.exp(3.0) + 1.0), 1.0 / (np.exp(3.0) + 1.0)]], rtol=1e-15)
    # unselected logits do not enter; shifting all logits changes nothing
    S2 = S.copy()
    S2[0, 0] = 100.0
    assert np.array_equal(softmax_selected(S2, I), w)
    assert np.allclose(softmax_selected(S + 7.5, I), w, rtol=1e-15)
    rng = np.random.default_rng(1)
    S = rng.standard_normal((50, 8))
    I = topk_stable(S, 3)
    assert np.allclose(softmax_selected(S, I).sum(1), 1.0, rtol=1e-15)
    assert np.array_equal(softmax_selected(S, topk_stable(S, 1)), np.ones((50, 1)))


def test_dispatch_lists_each_pair_once_in_token_order():
    rng = np.random.default_rng(2)
    E, k = 8, 2
    I = topk_stable(rng.standard_normal((100, E)), k)
    tokens, slots, start = dispatch(I, E)
    assert start[0] == 0 and start[-1] == 100 * k
    assert np.array_equal(np.diff(start), np.bincount(I.ravel(), minlength=E))
    pairs = set(zip(tokens.tolist(), slots.tolist()))
    assert pairs == {(t, s) for t in range(100) for s in range(k)}
    for e in range(E):
        rows = slice(start[e], start[e + 1])
        assert np.all(I[tokens[rows], slots[rows]] == e)
        assert np.all(np.diff(tokens[rows]) > 0)


def test_silu_closed_form():
    assert silu(np.array([0.0]))[0] == 0.0
    assert silu(np.array([np.log(3.0)]))[0] == pytest.approx(np.log(3.0) * 0.75, rel=1e-15)
    a = np.linspace(-20, 20, 81)
    assert np.allclose(silu(a), a * (0.5 * (1 + np.tanh(a / 2))), rtol=1e-13, atol=1e-15)
    assert np.allclose(silu(a) - silu(-a), a, atol=1e-12)        # a (s(a) + s(-a)) = a


def test_swiglu_written_out():
    rng = np.random.default_rng(3)
    n, dm, ffn = 3, 4, 5
    x, W1, W3, W2 = (_bf16(rng.standard_normal(s)) for s in ((n, dm), (ffn, dm), (ffn, dm), (dm, ffn)))
    want = np.empty((n, dm))
    for t in range(n):
        h = np.empty(ffn)
        for f in range(ffn):
            a = round_to(np.array([sum(x[t, j] * W1[f, j] for j in range(dm))]), "bf16")[0]
            b = round_to(np.array([sum(x[t, j] * W3[f, j] for j in range(dm))]), "bf16")[0]
            h[f] = round_to(np.array([a / (1 + np.exp(-a)) * b]), "bf16")[0]
        for o in range(dm):
            want[t, o] = sum(h[f] * W2[o, f] for f in range(ffn))
    assert np.array_equal(swiglu_expert(x, W1, W3, W2), round_to(want, "bf16"))


def _layer_weights(rng, E, dm, ffn):
    return (_bf16(rng.standard_normal((E, dm)) / np.sqrt(dm)),
            _bf16(rng.standard_normal((E, ffn, dm)) / np.sqrt(dm)),
            _bf16(rng.standard_normal((E, ffn, dm)) / np.sqrt(dm)),
            _bf16(rng.standard_normal((E, dm, ffn)) / np.sqrt(ffn)))


def test_identical_experts_give_one_expert():
    rng = np.random.default_rng(4)
    E, dm, ffn, k = 4, 8, 6, 2
    Wr, W1, W3, W2 = _layer_weights(rng, E, dm, ffn)
    W1[:] = W1[0]
    W3[:] = W3[0]
    W2[:] = W2[0]
    x = _bf16(rng.standard_normal((20, dm)))
    y, S, I, w = moe_layer(x, Wr, W1, W3, W2, k)
    assert np.allclose(y, swiglu_expert(x, W1[0], W3[0], W2[0]), rtol=2 ** -7, atol=1e-12)


def test_equal_logits_route_to_the_first_experts_evenly():
    rng = np.random.default_rng(5)
    E, dm, ffn, k = 8, 8, 4, 2
    _, W1, W3, W2 = _layer_weights(rng, E, dm, ffn)
    x = _bf16(rng.standard_normal((10, dm)))
    y, S, I, w = moe_layer(x, np.zeros((E, dm)), W1, W3, W2, k)
    assert np.all(I == [0, 1]) and np.all(w == 0.5)
    want = 0.5 * swiglu_expert(x, W1[0], W3[0], W2[0]) + 0.5 * swiglu_expert(x, W1[1], W3[1], W2[1])
    assert np.array_equal(y, round_to(want, "bf16"))


def test_combine_places_weighted_outputs():
    """Experts whose output is a constant c_e on every coordinate (W2 row sums
    picked so): y = sum_i w_i c_{I_i}, plus the shared expert's output."""
    rng = np.random.default_rng(6)
    E, dm, ffn, k, N = 4, 4, 2, 2, 30
    Wr = _bf16(rng.standard_normal((E, dm)))
    x = _bf16(np.abs(rng.standard_normal((N, dm))) + 1.0)
    # W1 = W3 = e_0: a = b = x_0 > 0 in both ffn rows; W2 picks coordinate 0 of h
    W1 = np.zeros((E, ffn, dm))
    W1[:, :, 0] = 1.0
    W3 = W1.copy()
    W2 = np.zeros((E, dm, ffn))
    W2[:, :, 0] = 1.0
    W2 *= np.arange(1, E + 1)[:, None, None]
    y, S, I, w = moe_layer(x, Wr, W1, W3, W2, k)
    h = round_to(silu(x[:, 0]) * x[:, 0], "bf16")
    for t in range(N):
        want = sum(w[t, s] * round_to(np.array([h[t] * (I[t, s] + 1)]), "bf16")[0] for s in range(k))
        assert np.all(y[t] == round_to(np.array([want]), "bf16")[0])
    ys, *_ = moe_layer(x, Wr, W1, W3, W2, k, shared=(W1[0], W3[0], W2[0]))
    assert np.allclose(ys, y + round_to(h, "bf16")[:, None], rtol=2 ** -7)


def test_router_is_a_bf16_linear():
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((5, 16)))
    Wr = _bf16(rng.standard_normal((8, 16)))
    S = router_logits(x, Wr)
    assert np.array_equal(S, round_to(x @ Wr.T, "bf16"))
    assert S.shape == (5, 8)


def test_lite_moe_shape_from_the_pages():
    lite = json.load(open(os.path.join(GOLDEN, "gpt_oss_lite_moe.json")))
    assert lite["experts"] == 8 and lite["top_k"] == 2 and lite["ffn_dim"] == 1536
    assert lite["shared_experts"] == 1 and lite["d_model"] == 768
