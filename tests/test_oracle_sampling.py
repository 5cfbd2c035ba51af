"""Pins for the oracle's sampling controls (oracle/sampling.py): hand-worked
penalty arithmetic and its order, greedy ties, closed-form distributions
(logits = log p at T = 1), each truncation on a worked example including
ties and the top-k-then-top-p renormalisation, and the draw's defining
property (over an even grid of u the tokens come out in proportion to their
kept probability)."""
import numpy as np
import pytest

from oracle.sampling import (kept_mask, probabilities, processed_logits, sample,
                             token_counts)

def _keep(p, **kw):
    args = dict(top_k=0, top_p=1.0, min_p=0.0)
    args.update(kw)
    z = np.log(np.asarray(p, np.float64)).astype(np.float32)
    return np.flatnonzero(kept_mask(z, 1.0, **args)).tolist()


def test_penalties_hand_worked():
    z = np.array([2.0, -2.0, 1.0, 0.5], np.float32)
    counts = np.array([1, 2, 0, 3])
    zp = processed_logits(z, None, counts, rep=2.0, presence=0.5, frequency=0.25)
    # seen & positive: /2; seen & negative: *2; unseen untouched; then -0.5, -0.25 c
    assert zp.tolist() == [2 / 2 - 0.5 - 0.25, -2 * 2 - 0.5 - 0.5, 1.0, 0.5 / 2 - 0.5 - 0.75]
    assert zp.dtype == np.float32


def test_penalties_off_and_bias_first():
    rng = np.random.default_rng(0)
    z = rng.standard_normal(100).astype(np.float32)
    c = rng.integers(0, 3, 100)
    assert np.array_equal(processed_logits(z, None, c, 1.0, 0.0, 0.0), z)
    # bias enters before the repetition penalty: (-1 + 2) / 2, not -1 * 2 + 2
    out = processed_logits(np.array([-1.0], np.float32), np.array([2.0], np.float32), [1], 2.0, 0.0, 0.0)
    assert out.tolist() == [0.5]
    # -inf bias masks a token whatever the penalties do
    out = processed_logits(np.array([3.0], np.float32), np.array([-np.inf], np.float32), [4], 1.3, 0.2, 0.1)
    assert out[0] == -np.inf


def test_fp32_rounding_of_each_step():
    # 1/3 is not a float: the division is rounded once to fp32, as is f*c
    z = np.array([1.0], np.float32)
    out = processed_logits(z, None, [3], 3.0, 0.0, 0.1)
    want = np.float32(np.float32(1.0) / np.float32(3.0)) - np.float32(np.float32(0.1) * np.float32(3))
    assert out[0] == np.float32(want)


def test_token_counts():
    h = [5, 1, 5, -1, 7, 5, 9]
    c = token_counts(h, 8)
    assert c.tolist() == [0, 1, 0, 0, 0, 3, 0, 1]           # -1 and 9 (>= V) ignored


def test_greedy_ties_and_empty_rows():
    z = np.array([1.0, 3.0, 3.0, 2.0], np.float32)
    tok, _, _ = sample(z, None, np.zeros(4), 1, 0, 0, 0.0, 0, 1.0, 0.0, 0.99)
    assert tok == 1
    tok, _, _ = sample(np.full(4, -np.inf, np.float32), None, np.zeros(4), 1, 0, 0, 0.7, 0, 1.0, 0.0, 0.5)
    assert tok == -1
    tok, _, _ = sample(np.full(4, -np.inf, np.float32), None, np.zeros(4), 1, 0, 0, 0.0, 0, 1.0, 0.0, 0.5)
    assert tok == -1


def test_softmax_closed_form():
    p = np.array([0.5, 0.3, 0.15, 0.05])
    assert np.allclose(probabilities(np.log(p), 1.0), p, rtol=1e-15)
    # T halves the log-probabilities: p^(1/T) renormalised
    q = p ** 2 / (p ** 2).sum()
    assert np.allclose(probabilities(np.log(p), 0.5), q, rtol=1e-14)


def test_top_k_keeps_ties():
    assert _keep([0.5, 0.3, 0.15, 0.05], top_k=2) == [0, 1]
    assert _keep([0.4, 0.2, 0.2, 0.2], top_k=2) == [0, 1, 2, 3]    # 2nd is tied: all kept
    assert _keep([0.1, 0.2, 0.3, 0.4], top_k=1) == [3]
    assert _keep([0.5, 0.3, 0.15, 0.05], top_k=4) == [0, 1, 2, 3]


def test_top_p_smallest_set():
    p = [0.5, 0.3, 0.15, 0.05]
    assert _keep(p, top_p=0.45) == [0]
    assert _keep(p, top_p=0.75) == [0, 1]
    assert _keep(p, top_p=0.81) == [0, 1, 2]
    assert _keep(p, top_p=0.99) == [0, 1, 2, 3]
    assert _keep([0.2, 0.4, 0.2, 0.2], top_p=0.5) == [0, 1, 2, 3]   # crossing inside a tie group
    assert _keep([0.2, 0.6, 0.1, 0.1], top_p=0.7) == [0, 1]


def test_top_p_renormalised_over_top_k():
    p = [0.4, 0.3, 0.2, 0.1]
    # over the top-2 mass 0.7 the first token's share is 4/7 > 0.55: one token
    assert _keep(p, top_k=2, top_p=0.55) == [0]
    # over the whole mass 0.4 < 0.55 would have kept two
    assert _keep(p, top_p=0.55) == [0, 1]


def test_min_p_relative_to_the_max():
    p = [0.5, 0.3, 0.15, 0.05]
    assert _keep(p, min_p=0.25) == [0, 1, 2]       # p >= 0.125
    assert _keep(p, min_p=0.35) == [0, 1]          # p >= 0.175
    assert _keep(p, min_p=1.0) == [0]
    assert _keep([0.25, 0.25, 0.25, 0.25], min_p=1.0) == [0, 1, 2, 3]


def test_truncations_intersect():
    p = [0.3, 0.05, 0.25, 0.15, 0.1, 0.15]
    assert _keep(p, top_k=4, min_p=0.6) == [0, 2]
    assert _keep(p, top_k=2, top_p=0.99) == [0, 2]
    assert _keep(p, top_p=0.5, min_p=0.1) == [0, 2]


def test_draw_frequencies_follow_the_kept_distribution():
    p = np.array([0.05, 0.3, 0.15, 0.5])
    z = np.log(p).astype(np.float32)
    n = 20000
    for kw, kept in ((dict(top_k=0, top_p=1.0, min_p=0.0), [0, 1, 2, 3]),
                     (dict(top_k=2, top_p=1.0, min_p=0.0), [1, 3]),
                     (dict(top_k=0, top_p=1.0, min_p=0.4), [1, 3])):
        toks = [sample(z, None, np.zeros(4), 1, 0, 0, 1.0, kw["top_k"], kw["top_p"], kw["min_p"],
                       (j + 0.5) / n)[0] for j in range(n)]
        freq = np.bincount(toks, minlength=4) / n
        want = np.zeros(4)
        want[kept] = p[kept] / p[kept].sum()
        assert np.allclose(freq, want, atol=2.0 / n)


def test_draw_inverts_in_id_order():
    p = np.array([0.1, 0.6, 0.3])
    z = np.log(p).astype(np.float32)
    args = (None, np.zeros(3), 1, 0, 0, 1.0, 0, 1.0, 0.0)
    assert sample(z, *args, 0.0)[0] == 0
    assert sample(z, *args, 0.0999)[0] == 0
    assert sample(z, *args, 0.1001)[0] == 1
    assert sample(z, *args, 0.6999)[0] == 1
    assert sample(z, *args, 0.7001)[0] == 2
    assert sample(z, *args, 0.999999)[0] == 2


def test_top_k_one_is_greedy_for_any_u():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(1000).astype(np.float32)
    for u in (0.0, 0.3, 0.999):
        assert sample(z, None, np.zeros(1000), 1, 0, 0, 0.8, 1, 1.0, 0.0, u)[0] == int(np.argmax(z))


@pytest.mark.parametrize("T", [0.2, 1.0, 3.0])
def test_low_temperature_limit_and_no_truncation(T):
    rng = np.random.default_rng(4)
    z = rng.standard_normal(500).astype(np.float32)
    keep = kept_mask(z, T, 0, 1.0, 0.0)
    assert keep.all()
    p = probabilities(z, T)
    assert np.isclose(p.sum(), 1.0, rtol=1e-14) and np.argmax(p) == np.argmax(z)
    pt = probabilities(z, 1e-3)
    assert pt[np.argmax(z)] > 0.999


def test_example_request_settings_from_the_pages():
    import json
    import os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sampling_example.json")))
    assert ex["vocab"] == 128000
    assert (ex["temperature"], ex["top_p"], ex["min_p"]) == (0.2, 0.95, 0.05)
    # at these settings a 128k-token row keeps only tokens near the top: min-p bounds the
    # kept logits to within T ln(1 / min_p) of the largest
    rng = np.random.default_rng(5)
    z = rng.standard_normal(ex["vocab"]).astype(np.float32)
    keep = kept_mask(z, ex["temperature"], 0, ex["top_p"], ex["min_p"])
    assert np.all(z[keep] >= z.max() - ex["temperature"] * np.log(1 / ex["min_p"]) - 1e-6)
    assert 1 <= keep.sum() < 100
