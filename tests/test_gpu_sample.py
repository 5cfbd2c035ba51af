"""GPU parity of the sampling controls (sample_tokens, sample_count_tokens)
against the oracle (oracle/sampling.py).

  * processed logits: bit-exact (the same fp32 operations in the same
    order);
  * greedy tokens and top-k sets: bit-exact (decided on exact fp32 logits,
    ties to the lower id / kept whole);
  * sampled tokens and kept counts: equal to the oracle's.  The oracle
    decides top-p, min-p and the draw in fp64 and the kernel in fp32
    weights with exact integer sums, so where an fp64 boundary sits within
    1e-5 (relative) of the decision the test accepts any token and count the
    oracle gives with top_p, min_p and u moved by that much, and such rows
    must stay rare;
  * counts: bit-exact (integer atomics).
Every call runs twice and must give the same tokens (determinism).
"""
import itertools

import numpy as np
import pytest
import torch

from oracle.sampling import kept_mask, processed_logits, sample, token_counts
from workloads import SAMPLE_B, SAMPLE_V, sampling_inputs

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")

DELTA = 1e-5


def _f32(x):
    """The value a float field of sa_sample_params carries."""
    return float(np.float32(x))


def _oracle_row(z, bias, counts, p, u):
    return sample(z, bias, counts, p["repetition"], p["presence"], p["frequency"], _f32(p["temperature"]),
                  p["top_k"], _f32(p["top_p"]), _f32(p["min_p"]), float(u))


def _near_variants(z, bias, counts, p, u):
    """(token, kept count) of the oracle with top_p, min_p, u moved by DELTA."""
    out = set()
    for dp, dm, du in itertools.product((-1, 0, 1), repeat=3):
        q = dict(p)
        if q["top_p"] < 1.0:
            q["top_p"] = min(1.0, _f32(q["top_p"]) * (1 + dp * DELTA))
        q["min_p"] = _f32(q["min_p"]) * (1 + dm * DELTA)
        uu = min(max(float(u) + du * DELTA, 0.0), np.nextafter(1.0, 0.0))
        tok, _, keep = _oracle_row(z, bias, counts, q, uu)
        out.add((tok, int(keep.sum()) if keep is not None else (1 if tok >= 0 else 0)))
    return out


def _run(logits, rows, u, bias=None, counts=None, update=False):
    B, V = logits.shape
    params = sa.sample_params(B, **{k: [r[k] for r in rows] for k in rows[0]})
    lg = torch.from_numpy(logits).cuda()
    ut = torch.from_numpy(np.asarray(u, np.float32)).cuda()
    bt = torch.from_numpy(bias).cuda() if bias is not None else None
    ct = torch.from_numpy(counts.astype(np.int32)).cuda() if counts is not None else None
    tok, kept, proc = sa.sample_tokens(lg, params, ut, bias=bt, counts=ct, update_counts=update,
                                       want_kept=True, want_processed=True)
    if not update:
        tok2 = sa.sample_tokens(lg, params, ut, bias=bt, counts=ct)
        assert torch.equal(tok, tok2)                     # deterministic
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), kept.cpu().numpy(), proc.cpu().numpy(),
            ct.cpu().numpy() if ct is not None else None)


def _params(**kw):
    p = dict(temperature=1.0, top_k=0, top_p=1.0, min_p=0.0, repetition=1.0, presence=0.0, frequency=0.0)
    p.update(kw)
    return p


def _check(logits, rows, u, bias=None, counts=None, max_near=1):
    B, V = logits.shape
    tok, kept, proc, _ = _run(logits, rows, u, bias, counts)
    near = 0
    for b in range(B):
        cb = counts[b] if counts is not None else np.zeros(V, np.int64)
        bb = None if bias is None else (bias if bias.ndim == 1 else bias[b])
        want_tok, zp, keep = _oracle_row(logits[b], bb, cb, rows[b], u[b])
        assert np.array_equal(proc[b].view(np.uint32), zp.view(np.uint32)), "row %d processed logits" % b
        want_kept = int(keep.sum()) if keep is not None else (1 if want_tok >= 0 else 0)
        if (tok[b], kept[b]) != (want_tok, want_kept):
            assert (int(tok[b]), int(kept[b])) in _near_variants(logits[b], bb, cb, rows[b], u[b]), \
                "row %d: got (%d, %d), oracle (%d, %d)" % (b, tok[b], kept[b], want_tok, want_kept)
            near += 1
    assert near <= max_near
    return tok, kept


# the example request's settings on the pages' vocabulary, penalties on
PAGE = dict(temperature=0.2, top_p=0.95, min_p=0.05)


def test_page_example_settings_full_vocab():
    d = sampling_inputs(SAMPLE_B, SAMPLE_V, seed=1)
    counts = np.stack([token_counts(h, SAMPLE_V) for h in d["history"]])
    rows = [_params(**PAGE, repetition=1.1, presence=0.2, frequency=0.1) for _ in range(SAMPLE_B)]
    tok, kept = _check(d["logits"], rows, d["u"], bias=None, counts=counts)
    assert np.all(kept >= 1)


@pytest.mark.parametrize("V", [1, 63, 4096, 10000, SAMPLE_V])
def test_greedy_and_ties(V):
    d = sampling_inputs(4, V, seed=2, bf16_logits=True)
    z = d["logits"].copy()
    z[1, :] = z[1, 0]                                  # all equal: token 0
    z[2, V // 2:] = z[2].max()                         # tie at the max: lowest id wins
    z[3, :] = -np.inf                                  # no token
    rows = [_params(temperature=0.0) for _ in range(4)]
    tok, kept = _check(z, rows, d["u"], max_near=0)
    assert tok[1] == 0 and tok[3] == -1 and kept[3] == 0
    assert tok[2] == min(int(np.argmax(z[2])), V // 2)


MIXED = [
    _params(temperature=0.7, top_k=50),
    _params(temperature=1.0, top_k=1),
    _params(temperature=1.3, top_p=0.9),
    _params(temperature=0.5, min_p=0.1),
    _params(temperature=1.0, top_k=40, top_p=0.8, min_p=0.02),
    _params(temperature=0.0),
    _params(temperature=2.0),                          # no truncation: the whole row
    _params(temperature=0.9, top_k=3000, top_p=0.99),
]


@pytest.mark.parametrize("V,seed", [(10000, 3), (SAMPLE_V, 4), (5000, 5)])
def test_mixed_rows(V, seed):
    d = sampling_inputs(len(MIXED), V, seed=seed, scale=1.5)
    _check(d["logits"], MIXED, d["u"], bias=d["bias"][:V])


@pytest.mark.parametrize("bf16", [False, True])
def test_large_kept_sets_take_the_radix_path(bf16):
    """Kept sets beyond the 4096 LDS candidates: top-k of 20000, top-p over a
    flat row (T = 3), both, and no truncation."""
    rows = [_params(temperature=1.0, top_k=20000), _params(temperature=3.0, top_p=0.9),
            _params(temperature=2.0, top_k=50000, top_p=0.7), _params(temperature=1.0),
            _params(temperature=1.5, top_k=10000, min_p=1e-6)]
    d = sampling_inputs(len(rows), SAMPLE_V, seed=6, scale=1.0, bf16_logits=bf16)
    tok, kept = _check(d["logits"], rows, d["u"])
    assert kept[0] >= 20000 and kept[3] == SAMPLE_V and kept[1] > 4096


@pytest.mark.parametrize("bf16", [False, True])
def test_edge_bucket_path(bf16):
    """One truncation rule on, more than 4096 tokens at or above its bucket,
    at most 4096 in the bucket itself (the full vocabulary, logits of scale
    2): the bucket alone is gathered and sorted, the histogram and per-chunk
    sums supply what lies above it, and the draw stays in one chunk."""
    rows = [_params(temperature=1.0, top_p=0.9), _params(temperature=0.8, top_k=8000),
            _params(temperature=1.5, top_p=0.99), _params(temperature=1.0, top_k=5000),
            _params(temperature=0.6, top_p=0.97), _params(temperature=2.0, top_k=30000)]
    d = sampling_inputs(len(rows), SAMPLE_V, seed=16, scale=2.0, bf16_logits=bf16)
    tok, kept = _check(d["logits"], rows, d["u"])
    assert kept[1] >= 8000 and kept[3] >= 5000 and kept[0] > 4096


def test_dense_buckets_take_the_radix_path():
    """Logits packed into a few buckets (1.5 + 0.05 N(0, 1)): the bound's
    bucket holds more than 4096 tokens, so single-rule rows too descend the
    radix levels."""
    rows = [_params(temperature=1.0, top_p=0.9), _params(temperature=0.5, top_k=30000),
            _params(temperature=0.05, top_p=0.5), _params(temperature=1.0, top_k=100)]
    d = sampling_inputs(len(rows), SAMPLE_V, seed=17, scale=1.0)
    logits = (1.5 + 0.05 * d["logits"]).astype(np.float32)
    tok, kept = _check(logits, rows, d["u"])
    assert kept[1] >= 30000 and kept[3] >= 100


def test_ties_are_kept_whole():
    """bf16 logits: many equal values; top-k and top-p keep the tie group."""
    V = 20000
    d = sampling_inputs(6, V, seed=7, scale=1.0, bf16_logits=True)
    rows = [_params(temperature=1.0, top_k=k) for k in (1, 2, 7, 100, 1000, 5000)]
    tok, kept = _check(d["logits"], rows, d["u"], max_near=0)
    for b, k in enumerate((1, 2, 7, 100, 1000, 5000)):
        vk = np.sort(d["logits"][b])[::-1][k - 1]
        assert kept[b] == int(np.count_nonzero(d["logits"][b] >= vk)) >= k


def test_draw_follows_u():
    """One row, many uniforms: every token equals the oracle's."""
    V, n = 3000, 64
    d = sampling_inputs(1, V, seed=8, scale=1.0)
    z = np.repeat(d["logits"], n, axis=0)
    u = (np.arange(n, dtype=np.float64) + 0.37) / n
    rows = [_params(temperature=0.8, top_p=0.95) for _ in range(n)]
    tok, _ = _check(z, rows, u.astype(np.float32), max_near=2)
    assert len(set(tok.tolist())) > 10


def test_penalties_bias_and_count_updates():
    V = 9000
    d = sampling_inputs(4, V, seed=9, history=500)
    counts = np.stack([token_counts(h, V) for h in d["history"]])
    bias2 = np.stack([d["bias"][:V], -d["bias"][:V], np.zeros(V, np.float32), d["bias"][:V] * 3])
    bias2[2, 17] = np.inf * -1                          # a masked token
    rows = [_params(temperature=0.6, repetition=1.3), _params(temperature=0.0, presence=1.5),
            _params(temperature=1.1, frequency=0.7, top_k=100), _params(temperature=0.9, repetition=0.8,
                                                                        presence=-0.5, frequency=0.25)]
    _check(d["logits"], rows, d["u"], bias=bias2, counts=counts)
    tok, _, _, ct = _run(d["logits"], rows, d["u"], bias=bias2, counts=counts, update=True)
    want = counts.copy()
    for b in range(4):
        want[b, tok[b]] += 1
    assert np.array_equal(ct, want)


def test_count_tokens_matches_oracle():
    B, V, H = 5, 128000, 3000
    rng = np.random.default_rng(10)
    ids = rng.integers(-5, V + 5, size=(B, H)).astype(np.int32)
    ids[:, :100] = 7                                    # many repeats
    counts = torch.zeros((B, V), dtype=torch.int32, device="cuda")
    sa.sample_count_tokens(torch.from_numpy(ids).cuda(), counts)
    sa.sample_count_tokens(torch.from_numpy(ids).cuda(), counts)   # adds
    got = counts.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b], 2 * token_counts(ids[b], V))


def test_invalid_rows_get_no_token():
    V = 1000
    d = sampling_inputs(6, V, seed=11)
    rows = [_params(temperature=-1.0), _params(top_p=0.0), _params(min_p=1.5), _params(repetition=0.0),
            _params(temperature=1.0), _params(temperature=0.7, top_k=-3)]
    u = d["u"].copy()
    u[4] = 1.0                                          # u outside [0, 1)
    tok, kept, _, _ = _run(d["logits"], rows, u)
    assert np.all(tok == -1) and np.all(kept == 0)


def test_strided_rows_through_the_c_abi():
    """logits rows padded to a wider stride (the C-ABI's logits_stride), a
    bias row shared through stride 0, odd vocabulary sizes."""
    from long_context_sparse_yarn_amd import _binding as B
    for V, pad in ((1, 3), (5, 0), (4097, 37), (10001, 64)):
        Bn = 3
        d = sampling_inputs(Bn, V, seed=12, scale=1.0)
        stride = V + pad
        wide = np.full((Bn, stride), np.nan, np.float32)
        wide[:, :V] = d["logits"]
        rows = [_params(temperature=0.0), _params(temperature=0.9, top_p=0.8), _params(temperature=1.2, top_k=3)]
        params = sa.sample_params(Bn, **{k: [r[k] for r in rows] for k in rows[0]})
        lg = torch.from_numpy(wide).cuda()
        bias = torch.from_numpy(d["bias"][:V]).cuda()
        ut = torch.from_numpy(d["u"]).cuda()
        tok = torch.empty(Bn, dtype=torch.int32, device="cuda")
        kept = torch.empty(Bn, dtype=torch.int32, device="cuda")
        nb = sa.sample_workspace_bytes(Bn, V)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        st = B._sample_tokens(lg.data_ptr(), Bn, V, stride, bias.data_ptr(), 0, None, params.data_ptr(),
                              ut.data_ptr(), 0, tok.data_ptr(), kept.data_ptr(), None, ws.data_ptr(), nb,
                              torch.cuda.current_stream().cuda_stream)
        assert st == 0, B.last_error()
        torch.cuda.synchronize()
        for b in range(Bn):
            want, _, keep = _oracle_row(d["logits"][b], d["bias"][:V], np.zeros(V, np.int64), rows[b], d["u"][b])
            assert int(tok[b]) == want
            assert int(kept[b]) == (int(keep.sum()) if keep is not None else 1)


def test_large_batch_several_chunks_per_histogram_workgroup():
    """96 rows of the full vocabulary: the histogram launch gives each
    workgroup several chunks of a row; every path (min-p candidates, gather,
    radix levels, chunk-mass draw, greedy) in one batch."""
    B = 96
    rows = [dict(r) for r in (MIXED + [_params(**PAGE)]) * (B // (len(MIXED) + 1) + 1)][:B]
    d = sampling_inputs(B, SAMPLE_V, seed=13, scale=1.5)
    _check(d["logits"], rows, d["u"], max_near=2)


@pytest.mark.parametrize("seed", [21, 22, 23, 24])
def test_random_settings_sweep(seed):
    """16 rows of random settings (temperature, top-k, top-p, min-p, the three
    penalties, bias on or off) over a random vocabulary size, bf16-rounded or
    fp32 logits: every row against the oracle."""
    rng = np.random.default_rng(seed)
    V = int(rng.integers(300, 40000))
    B = 16
    d = sampling_inputs(B, V, seed=seed, scale=float(rng.uniform(0.5, 4.0)), history=200,
                        bf16_logits=bool(seed % 2))
    counts = np.stack([token_counts(h, V) for h in d["history"]])
    rows = []
    for _ in range(B):
        T = 0.0 if rng.random() < 0.15 else float(rng.uniform(0.05, 2.5))
        rows.append(_params(temperature=T,
                            top_k=int(rng.choice([0, 1, 5, 50, 500, V // 2, V + 3])),
                            top_p=float(rng.choice([1.0, 0.5, 0.9, 0.99, 0.999])),
                            min_p=float(rng.choice([0.0, 0.0, 0.01, 0.1, 0.5])),
                            repetition=float(rng.choice([1.0, 1.2, 0.9])),
                            presence=float(rng.choice([0.0, 0.3, -0.2])),
                            frequency=float(rng.choice([0.0, 0.05]))))
    bias = d["bias"][:V] if seed % 3 else None
    _check(d["logits"], rows, d["u"], bias=bias, counts=counts, max_near=1)
