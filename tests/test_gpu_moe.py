"""GPU parity of the MoE layer (moe_route, moe_dispatch, moe_layer) against the
oracle (oracle/moe.py).  The oracle routes every token by itself, from its
own fp64 logits; nothing the kernel computes is fed into it.

  * router logits: the kernel sums d_model exact bf16 products in fp32 and
    rounds once to bf16.  Its bf16 logit must be one of the roundings of a
    value within eps = 2^-20 * sum_i |x_i w_i| of the exact logit (checked for
    every logit), within one ulp of the oracle's, and bit-equal for > 99%.
  * routing ids (an integer decision taken from floating point, "MoE-Xtend"
    README, MOE ROUTING: ties broken consistently): given those admissible
    roundings, the oracle marks a token undecided when two experts it ranks
    a above b (a among its top k) could swap places -- b's highest
    admissible logit above a's lowest, or equal to it with b the lower id.
    Every other token is decided and the kernel's ids must equal the
    oracle's bit for bit.  Undecided tokens must stay rare (<= 0.2%, or
    one token of a small case); on them the kernel's ids must be a valid
    top-k of its own logits (largest first, equal logits to the lower id).
    Experts with identical weight rows compute identical sums, so their
    exact ties are decided (to the lower id) and checked exactly.
  * dispatch: rows and expert starts bit-exact;
  * layer: the oracle layer on its own routing; compared on every token the
    kernel routed as the oracle did (all decided tokens).  Each bf16 rounding
    point (gate, up, gated product, expert output) may sit one ulp from the
    oracle's where the fp32 sum lands near a midpoint, so y is held to
    |got - want| <= 2^-6 (|want| + rms(want)), with > 99% of elements within
    one ulp.
"""
import numpy as np
import pytest
import torch

from oracle.moe import dispatch, moe_layer, router_logits, softmax_selected, topk_stable
from oracle.rounding import round_to
from workloads import bf16_round
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _w(rng, shape, fan_in):
    return bf16_round((rng.standard_normal(shape) / np.sqrt(fan_in)).astype(np.float32))


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().astype(np.int64)


ROUTE_CASES = [(300, 64, 8, 2), (1000, 768, 8, 2), (77, 128, 32, 4), (50, 64, 64, 8), (64, 192, 5, 3)]
LOGIT_EPS = 2.0 ** -20          # kernel fp32 sum within LOGIT_EPS * sum|x_i w_i| of the exact logit


def routing_ranges(x, Wr):
    """Oracle side: exact fp64 logits and, per logit, the lowest and highest
    bf16 value a sum within the error bound can round to."""
    xs, ws = np.asarray(x, np.float64), np.asarray(Wr, np.float64)
    exact = xs @ ws.T
    eps = LOGIT_EPS * (np.abs(xs) @ np.abs(ws).T)
    return exact, round_to(exact - eps, "bf16"), round_to(exact + eps, "bf16")


def undecided_tokens(S, lo, hi, Wr, k):
    """Tokens whose top-k (ids and their order) the admissible roundings
    could change, decided from the oracle's values alone."""
    N, E = S.shape
    same = np.array([[np.array_equal(Wr[a], Wr[b]) for b in range(E)] for a in range(E)])
    und = np.zeros(N, dtype=bool)
    for t in range(N):
        order = sorted(range(E), key=lambda e: (-S[t, e], e))
        for ia in range(k):
            a = order[ia]
            for b in order[ia + 1:]:
                if same[a, b]:
                    continue
                if hi[t, b] > lo[t, a] or (hi[t, b] == lo[t, a] and b < a):
                    und[t] = True
    return und


def check_routing(x, Wr, k, lg, ids):
    """Kernel logits lg [N, E] (as float64) and ids [N, k] against the
    oracle's own routing.  Returns (oracle ids, mask of tokens routed alike,
    number of undecided tokens)."""
    exact, lo, hi = routing_ranges(x, Wr)
    S = router_logits(x, Wr)
    I = topk_stable(S, k)
    assert np.all((lg >= lo) & (lg <= hi)), "a kernel logit outside its admissible roundings"
    und = undecided_tokens(S, lo, hi, Wr, k)
    N = S.shape[0]
    assert und.sum() <= max(1, int(0.002 * N)), "undecided tokens: %d of %d" % (und.sum(), N)
    same = np.all(ids == I, axis=1)
    assert np.all(same | und), "decided tokens routed differently: %s" % np.nonzero(~(same | und))[0][:8]
    for t in np.nonzero(und & ~same)[0]:          # a valid top-k of the kernel's own logits
        order = sorted(range(S.shape[1]), key=lambda e: (-lg[t, e], e))
        assert list(ids[t]) == order[:k]
    print("routing: %d tokens, %d undecided, %d routed differently" % (N, und.sum(), (~same).sum()))
    return I, same, int(und.sum())


@pytest.mark.parametrize("N,dm,E,k", ROUTE_CASES)
def test_route_matches_oracle(N, dm, E, k):
    rng = np.random.default_rng(N + dm + E)
    x = bf16_round(rng.standard_normal((N, dm)).astype(np.float32))
    Wr = _w(rng, (E, dm), dm)
    Wr[E - 1] = Wr[0]                       # equal logits for experts 0 and E-1
    logits, ids, w = sa.moe_route(dev(x, "bf16"), dev(Wr, "bf16"), k)
    torch.cuda.synchronize()
    want = router_logits(x, Wr)
    lg = host(logits).astype(np.float64)
    ulp = np.abs(_bits(logits) - _bits(torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16)))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.99
    got = ids.cpu().numpy().astype(np.int64)
    I, same, _ = check_routing(x, Wr, k, lg, got)
    # weights: the oracle's softmax over its own selected logits.  Where the
    # kernel's selected logits are the oracle's bit for bit the fp32 softmax
    # must agree to 1e-6; a one-ulp logit (<= 2^-7 relative) moves a weight
    # by at most w(1-w) 2^-7 |S| <= 2e-3 at these logit sizes.
    wk, wo = w.cpu().numpy(), softmax_selected(want, I)
    exact = same & np.all(np.take_along_axis(lg, I, 1) == np.take_along_axis(want, I, 1), axis=1)
    assert exact.mean() > 0.97
    assert np.abs(wk[exact] - wo[exact]).max() <= 1e-6
    assert np.abs(wk[same] - wo[same]).max() <= 2e-3
    assert np.all(want[:, 0] == want[:, E - 1])                       # the tie is real ...
    both = np.isin(I, [0]).any(1) & np.isin(I, [E - 1]).any(1)
    assert both.any()
    assert np.all((got == 0).argmax(1)[both] < (got == E - 1).argmax(1)[both])   # ... and 0 wins it


def test_route_all_equal_logits():
    N, dm, E, k = 40, 64, 8, 3
    x = bf16_round(np.random.default_rng(0).standard_normal((N, dm)).astype(np.float32))
    logits, ids, w = sa.moe_route(dev(x, "bf16"), dev(np.zeros((E, dm), np.float32), "bf16"), k)
    assert np.all(ids.cpu().numpy() == [0, 1, 2])
    assert np.all(np.abs(w.cpu().numpy() - 1.0 / 3.0) <= 1e-7)


@pytest.mark.parametrize("N,E,k", [(1000, 8, 2), (257, 64, 8), (513, 5, 1), (3, 4, 4)])
def test_dispatch_matches_oracle(N, E, k):
    rng = np.random.default_rng(N * E + k)
    # random distinct ids per token, skewed so one expert gets nothing
    p = np.ones(E)
    p[E // 2] = 0.0 if E > k else 1.0
    p /= p.sum()
    I = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(N)]).astype(np.int32)
    rows, start = sa.moe_dispatch(torch.from_numpy(I).cuda(), E)
    torch.cuda.synchronize()
    tokens, slots, st = dispatch(I.astype(np.int64), E)
    assert np.array_equal(start.cpu().numpy(), st)
    assert np.array_equal(rows.cpu().numpy(), tokens * k + slots)


def _layer(rng, N, dm, E, k, ffn, ffn_s):
    x = bf16_round(rng.standard_normal((N, dm)).astype(np.float32))
    Wr = _w(rng, (E, dm), dm)
    W1, W3 = _w(rng, (E, ffn, dm), dm), _w(rng, (E, ffn, dm), dm)
    W2 = _w(rng, (E, dm, ffn), ffn)
    sh = None
    if ffn_s:
        sh = (_w(rng, (ffn_s, dm), dm), _w(rng, (ffn_s, dm), dm), _w(rng, (dm, ffn_s), ffn_s))
    return x, Wr, W1, W3, W2, sh


def _run(x, Wr, W1, W3, W2, sh, k):
    w13 = dev(np.concatenate([W1, W3], axis=1), "bf16")
    shared = None
    if sh is not None:
        shared = (dev(np.concatenate([sh[0], sh[1]], axis=0), "bf16"), dev(sh[2], "bf16"))
    y = sa.moe_layer(dev(x, "bf16"), dev(Wr, "bf16"), w13, dev(W2, "bf16"), k, shared=shared)
    logits, ids, _ = sa.moe_route(dev(x, "bf16"), dev(Wr, "bf16"), k)
    torch.cuda.synchronize()
    return y, host(logits).astype(np.float64), ids.cpu().numpy().astype(np.int64)


def _check(y_dev, want):
    got = host(y_dev)
    assert np.all(np.isfinite(got))
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = np.abs(got - want)
    assert np.all(err <= 2.0 ** -6 * (np.abs(want) + rms)), float((err / (np.abs(want) + rms)).max())
    ulp = np.abs(_bits(y_dev) - _bits(torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16)))
    print("layer: %.4f of elements bit-equal, %.4f within one ulp, max %d ulp" % (
        (ulp == 0).mean(), (ulp <= 1).mean(), ulp.max()))
    assert (ulp <= 1).mean() > 0.99


LAYER_CASES = [
    # N, d_model, E, k, ffn, ffn_shared
    (300, 128, 8, 2, 256, 128),
    (600, 64, 4, 1, 128, 0),
    (257, 768, 8, 2, 1536, 1536),      # GPT-OSS-Lite widths, ragged token count
    (100, 192, 32, 4, 128, 0),
]


@pytest.mark.parametrize("N,dm,E,k,ffn,ffn_s", LAYER_CASES)
def test_moe_layer_matches_oracle(N, dm, E, k, ffn, ffn_s):
    rng = np.random.default_rng(N + dm + E + ffn)
    x, Wr, W1, W3, W2, sh = _layer(rng, N, dm, E, k, ffn, ffn_s)
    y, lg, ids = _run(x, Wr, W1, W3, W2, sh, k)
    want, _, I, _ = moe_layer(x, Wr, W1, W3, W2, k, shared=sh)       # the oracle's own routing
    I2, same, _ = check_routing(x, Wr, k, lg, ids)
    assert np.array_equal(I, I2)
    keep = torch.from_numpy(np.nonzero(same)[0]).cuda()
    _check(y[keep], want[same])


@pytest.mark.timeout(300)
def test_moe_layer_lite_full_size_sampled_tokens():
    """The GPT-OSS-Lite MoE shape (16384 tokens, d_model 768, 8 experts, top 2,
    SwiGLU ffn 1536, one shared expert) in the launch bench.py times.  The
    routing of every token is checked against the oracle's; the layer output
    on sampled tokens (tokens are routed independently, so the oracle takes
    the sampled rows alone, with its own routing)."""
    rng = np.random.default_rng(21)
    N, dm, E, k, ffn = 16384, 768, 8, 2, 1536
    x, Wr, W1, W3, W2, sh = _layer(rng, N, dm, E, k, ffn, ffn)
    y, lg, ids = _run(x, Wr, W1, W3, W2, sh, k)
    I, same, n_und = check_routing(x, Wr, k, lg, ids)
    toks = np.array(sorted(set([0, 1, 255, 256, N - 1] + list(rng.choice(N, 59, replace=False)))))
    toks = toks[same[toks]]
    want, _, I_s, _ = moe_layer(x[toks], Wr, W1, W3, W2, k, shared=sh)
    assert np.array_equal(I_s, I[toks])
    _check(y[torch.from_numpy(toks).cuda()], want)
    # every expert got work and the counts add up
    assert np.bincount(ids.ravel(), minlength=E).sum() == N * k
