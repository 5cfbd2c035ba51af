"""sinkattn_decode_noalloc (decode with the library's static per-GPU scratch,
for callers that cannot allocate) against sinkattn_decode with a caller
workspace: the same kernels, so the outputs must agree bit for bit, on two
calls in a row, the second with a smaller input (a scratch that keeps the
first call's partials must not leak into the second), plus a short band
span (no partials), and both against the fp64 oracle (2e-2)."""
import numpy as np
import pytest
import torch

from oracle.kvcache import OracleKVCache
from oracle.layer import decode_step
from workloads import Yarn, bf16_round
from tests.gpu_helpers import TOL, dev, host, lib_yarn, max_abs, oracle_tables

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _draw(rng, *shape):
    return bf16_round(rng.standard_normal(shape).astype(np.float32))


def _one(B, prefix, n_q, n_kv, d, W, seed):
    """Cache with `prefix` rows plus one decode token; both entry points on
    the same inputs; returns (noalloc out, workspace out, oracle out)."""
    rng = np.random.default_rng(seed)
    y = Yarn()
    sm = 1.0 / np.sqrt(d)
    C = ((prefix + 1 + 31) // 32) * 32 + 32
    pk, pv = _draw(rng, B, prefix, n_kv, d), _draw(rng, B, prefix, n_kv, d)
    q, k, v = _draw(rng, B, 1, n_q, d), _draw(rng, B, 1, n_kv, d), _draw(rng, B, 1, n_kv, d)
    sinks = rng.standard_normal(n_q).astype(np.float32)
    cache = sa.KVCache.empty(B, C, n_kv, d, fill=float("nan"))
    cache.append(dev(pk, "bf16"), dev(pv, "bf16"))
    ly = lib_yarn(d, y)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o = cache.offset
    sa.yarn_rope_apply(qd, o, ly)
    sa.yarn_rope_apply(kd, o, ly)
    cache.append(kd, vd)
    s_t = torch.from_numpy(sinks).cuda()
    got = sa.sinkattn_decode_noalloc(qd, cache, s_t, W, sm)
    ref = sa.sinkattn_decode(qd, cache, s_t, W, sm, workspace=sa.decode_workspace(cache, n_q))
    torch.cuda.synchronize()
    inv, c = oracle_tables(d, y)
    oc = OracleKVCache(B, C, n_kv, d)
    oc.append(pk.astype(np.float64), pv.astype(np.float64))
    want, _, _ = decode_step(oc, q, k, v, sinks, W, sm, inv, c, "bf16")
    return got, ref, want


@pytest.mark.parametrize("first,second", [
    ((2, 5000, 64, 8, 64, 0), (1, 1000, 16, 4, 96, 0)),      # split spans: 4.3 MB, then 0.2 MB
    ((1, 3000, 32, 8, 128, 0), (1, 300, 8, 2, 64, 128)),     # then a band span (no partials)
])
def test_noalloc_decode_matches_workspace_decode(first, second):
    for i, shape in enumerate((first, second)):
        got, ref, want = _one(*shape, seed=100 + i)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), shape
        assert np.all(np.isfinite(host(got)))
        assert max_abs(host(got), want) <= TOL["bf16"], shape
