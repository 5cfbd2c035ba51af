"""GPU parity of sinkattn_qkv_rope_append (the fused qkv projection with the
RoPE + append epilogue) against the oracle (oracle/qkv.py, then the layer
oracle's RoPE and append).

Tolerance: the kernel sums d_model products in fp32 in its own order, so
its bf16 projection can sit one bf16 ulp from the oracle's once-rounded
value where the exact sum is near a rounding midpoint (a small fraction of
elements).  V (no rotation): at most one ulp, almost all exact.  Q and K are
rotations of such values: |got - want| <= 2^-7 c (|u| + |v|) + 2^-7 |want|
with (u, v) the oracle's pair before rotation (one input ulp through the
rotation plus the output rounding on both sides), and almost all bit-exact.
Cache rows outside the append keep their NaN sentinels.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle.qkv import qkv_project, qkv_split, qkv_width
from oracle.rounding import round_to
from oracle.yarn import rope_apply, yarn_concentration
from workloads import Yarn, bf16_round
from tests.gpu_helpers import dev, host, lib_yarn, oracle_tables

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().astype(np.int64)


def _ulps(got_dev, want):
    w = torch.from_numpy(np.ascontiguousarray(want, np.float32)).to(torch.bfloat16)
    return np.abs(_bits(got_dev) - _bits(w))


def _inputs(rng, B, T, dm, n_q, n_kv, d):
    N = qkv_width(n_q, n_kv, d)
    x = bf16_round(rng.standard_normal((B, T, dm)).astype(np.float32))
    W = bf16_round((rng.standard_normal((N, dm)) / np.sqrt(dm)).astype(np.float32))
    b = bf16_round((0.1 * rng.standard_normal(N)).astype(np.float32))
    return x, W, b


def _oracle(x, W, b, n_q, n_kv, d, o, y):
    q, k, v = qkv_split(qkv_project(x, W, b), n_q, n_kv, d)
    inv, c = oracle_tables(d, y)
    return q, k, v, round_to(rope_apply(q, o, inv, c), "bf16"), round_to(rope_apply(k, o, inv, c), "bf16")


def _rot_tol(pre, want, c):
    """2^-7 c (|u| + |v|) + 2^-7 |want| per element of a rotated tensor."""
    d = pre.shape[-1]
    h = d // 2
    s = np.abs(pre[..., :h]) + np.abs(pre[..., h:])
    s = np.concatenate([s, s], -1)
    return 2.0 ** -7 * c * s + 2.0 ** -7 * np.abs(want)


def _check(got_q, got_k_rows, got_v_rows, q, k, v, q_rot, k_rot, c):
    for name, got, pre, want in (("q", got_q, q, q_rot), ("k", got_k_rows, k, k_rot)):
        g = host(got)
        assert np.all(np.isfinite(g)), name
        err = np.abs(g - want)
        assert np.all(err <= _rot_tol(pre, want, c)), (name, float(err.max()))
        assert (_ulps(got, want) == 0).mean() > 0.98, name
    u = _ulps(got_v_rows, v)
    assert u.max() <= 1 and (u == 0).mean() > 0.99


QKV_CASES = [
    # B, T, d_model, n_q, n_kv, d, prefix
    (1, 40, 128, 4, 2, 64, 0),          # one partial token tile
    (2, 130, 192, 8, 4, 96, 5),         # ragged tiles over two sequences, d = 96
    (1, 64, 256, 6, 1, 128, 33),        # d = 128, unaligned offset
    (1, 50, 64, 3, 1, 64, 0),           # odd number of heads: half-empty last tile
    (2, 33, 2880, 8, 1, 64, 7),         # gpt-oss width: 45 contraction stages
    (1, 257, 768, 8, 4, 96, 100),       # GPT-OSS-Lite width
]


@pytest.mark.parametrize("B,T,dm,n_q,n_kv,d,prefix", QKV_CASES)
def test_qkv_rope_append_matches_oracle(B, T, dm, n_q, n_kv, d, prefix):
    rng = np.random.default_rng(B * 7 + T + dm + d)
    y = Yarn()
    x, W, b = _inputs(rng, B, T, dm, n_q, n_kv, d)
    C = ((prefix + T + 31) // 32) * 32 + 32
    cache = sa.KVCache.empty(B, C, n_kv, d, fill=float("nan"))
    if prefix:
        pk = bf16_round(rng.standard_normal((B, prefix, n_kv, d)).astype(np.float32))
        cache.append(dev(pk, "bf16"), dev(pk, "bf16"))
    q_out = sa.qkv_rope_append(cache, dev(x, "bf16"), dev(W, "bf16"), dev(b, "bf16"), n_q,
                               lib_yarn(d, y))
    torch.cuda.synchronize()
    assert cache.offset == prefix + T
    q, k, v, q_rot, k_rot = _oracle(x, W, b, n_q, n_kv, d, prefix, y)
    rows = slice(prefix, prefix + T)
    _check(q_out, cache.k[:, rows], cache.v_rows()[:, rows], q, k, v, q_rot, k_rot,
           yarn_concentration(y.factor))
    # rows past the append keep their sentinels
    assert np.all(np.isnan(host(cache.k[:, prefix + T:])))
    assert np.all(np.isnan(host(cache.v_rows()[:, prefix + T:])))


def test_qkv_equals_projection_then_append_rope_qk():
    """The fused path against the library's separate path fed with the same
    bf16 projection computed by torch: equal within the tolerance above
    (the two fp32 summation orders differ), mostly bit for bit."""
    B, T, dm, n_q, n_kv, d = 2, 100, 512, 8, 2, 64
    rng = np.random.default_rng(5)
    y = Yarn()
    x, W, b = _inputs(rng, B, T, dm, n_q, n_kv, d)
    xd, Wd, bd = dev(x, "bf16"), dev(W, "bf16"), dev(b, "bf16")
    c1 = sa.KVCache.empty(B, 128, n_kv, d, fill=float("nan"))
    q1 = sa.qkv_rope_append(c1, xd, Wd, bd, n_q, lib_yarn(d, y))
    qkv = (xd.float() @ Wd.float().t() + bd.float()).to(torch.bfloat16)
    q, k, v = qkv[..., :n_q * d], qkv[..., n_q * d:(n_q + n_kv) * d], qkv[..., (n_q + n_kv) * d:]
    c2 = sa.KVCache.empty(B, 128, n_kv, d, fill=float("nan"))
    q2 = c2.append_rope_qk(q.reshape(B, T, n_q, d).contiguous(), k.reshape(B, T, n_kv, d).contiguous(),
                           v.reshape(B, T, n_kv, d).contiguous(), lib_yarn(d, y))
    torch.cuda.synchronize()
    c = yarn_concentration(y.factor)
    pre_q = host(q.reshape(B, T, n_q, d))
    pre_k = host(k.reshape(B, T, n_kv, d))
    for got, want, pre in ((q1, q2, pre_q), (c1.k[:, :T], c2.k[:, :T], pre_k)):
        err = np.abs(host(got) - host(want))
        assert np.all(err <= _rot_tol(pre, host(want), c))
        assert (_bits(got) == _bits(want)).mean() > 0.98
    assert (_bits(c1.v_rows()[:, :T]) == _bits(c2.v_rows()[:, :T])).mean() > 0.99


@pytest.mark.timeout(300)
@pytest.mark.parametrize("w,dm", [(wl.GPTOSS_PREFILL, 2880), (wl.LITE_PREFILL, 768)],
                         ids=["gptoss", "lite"])
def test_qkv_full_size_sampled_tokens(w, dm):
    """The workloads' shapes (gpt-oss: 8192 tokens, d_model 2880, 64/8/64;
    GPT-OSS-Lite: 4 x 4096 tokens, d_model 768, 8/4/96) in the launch bench.py
    times; the oracle checks every feature of sampled tokens, including tile
    edges."""
    rng = np.random.default_rng(11)
    x, W, b = _inputs(rng, w.B, w.T, dm, w.n_q, w.n_kv, w.d_h)
    cache = sa.KVCache.empty(w.B, w.capacity, w.n_kv, w.d_h, fill=float("nan"))
    q_out = sa.qkv_rope_append(cache, dev(x, "bf16"), dev(W, "bf16"), dev(b, "bf16"), w.n_q,
                               lib_yarn(w.d_h, w.yarn))
    torch.cuda.synchronize()
    toks = sorted(set([0, 1, 63, 64, 127, 128, w.T - 1] + list(rng.choice(w.T, 25, replace=False))))
    c = yarn_concentration(w.yarn.factor)
    for bi in range(w.B):
        xs = x[bi:bi + 1, toks]
        q, k, v = qkv_split(qkv_project(xs, W, b), w.n_q, w.n_kv, w.d_h)
        inv, cc = oracle_tables(w.d_h, w.yarn)
        pos = np.array(toks)
        q_rot = np.stack([round_to(rope_apply(q[:, i:i + 1], int(p), inv, cc), "bf16")[:, 0]
                          for i, p in enumerate(pos)], 1)
        k_rot = np.stack([round_to(rope_apply(k[:, i:i + 1], int(p), inv, cc), "bf16")[:, 0]
                          for i, p in enumerate(pos)], 1)
        _check(q_out[bi:bi + 1, toks], cache.k[bi:bi + 1, toks], cache.v_rows()[bi:bi + 1, toks],
               q, k, v, q_rot, k_rot, c)
