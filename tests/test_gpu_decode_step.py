"""GPU parity of sinkattn_decode_step, the fused decode step (RoPE of the
token's Q and K, append of its K/V row, sink attention in the same launch).

Against the separate calls it replaces -- kv_cache_append_rope_qk, then
sinkattn_decode -- bit for bit: the output, the rotated Q, and every K and V
row of the cache, over sweeps that cover both decode kernels (spans up to
256 rows in one workgroup per (b, g), longer spans split with a merge), every
head dimension, q_mult 1 to 16, the token's row at every position inside a
32-row block, the first token of an empty cache, full causal and band
layers, and a ring cache that wraps.  Against the fp64 oracle (its own RoPE,
append and attention from the raw draws) within 2e-2 on every step.
"""
import numpy as np
import pytest
import torch

from oracle.kvcache import OracleKVCache
from oracle.layer import decode_step
from oracle.ring import OracleRingCache, ring_decode
from workloads import Yarn, bf16_round
from tests.gpu_helpers import TOL, dev, host, lib_yarn, max_abs, oracle_rot, oracle_tables

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _draw(shape, rng):
    return bf16_round(rng.standard_normal(shape).astype(np.float32))


def _bits(t):
    return t.contiguous().view(torch.int16)


STEP_CASES = [
    # B, prefix, steps, n_q, n_kv, d, window
    (1, 0, 40, 8, 2, 64, 0),           # from an empty cache: rows 0..39, short kernel
    (2, 200, 40, 64, 8, 64, 0),        # short kernel up to 240 rows, then split + merge
    (2, 1000, 33, 64, 8, 64, 128),     # band: short kernel, every slot of a block
    (1, 3000, 6, 64, 8, 64, 0),        # split + merge, many splits
    (1, 320, 12, 8, 2, 64, 0),         # folded splits: 12 pieces over 11 blocks, one empty
    (3, 700, 5, 16, 1, 128, 0),        # q_mult 16, d 128
    (2, 250, 12, 24, 4, 96, 0),        # d 96, q_mult 6, across the short/split boundary
    (1, 77, 5, 8, 8, 96, 50),          # q_mult 1, band narrower than a block
    (1, 2000, 4, 32, 4, 128, 512),     # band wider than the short kernel's span
    (1, 600, 8, 16, 2, 64, 256),       # 256-row band: nine blocks (one wave walks three), then eight
]


def _caches(B, prefix, steps, n_kv, d, rng, C=None):
    if C is None:
        C = ((prefix + steps + 31) // 32) * 32 + 32
    pk = _draw((B, prefix, n_kv, d), rng)
    pv = _draw((B, prefix, n_kv, d), rng)
    pair = []
    for _ in range(2):
        c = sa.KVCache.empty(B, C, n_kv, d, fill=float("nan"))
        if prefix:
            c.append(dev(pk, "bf16"), dev(pv, "bf16"))
        pair.append(c)
    return pair, pk, pv


@pytest.mark.parametrize("B,prefix,steps,n_q,n_kv,d,W", STEP_CASES)
def test_decode_step_equals_separate_calls_and_oracle(B, prefix, steps, n_q, n_kv, d, W):
    rng = np.random.default_rng(1000 * d + prefix + W)
    y = Yarn()
    ly = lib_yarn(d, y)
    inv, conc = oracle_tables(d, y)
    sm = 1.0 / np.sqrt(d)
    sinks = rng.standard_normal(n_q).astype(np.float32)
    s_t = torch.from_numpy(sinks).cuda()
    (ca, cb), pk, pv = _caches(B, prefix, steps, n_kv, d, rng)
    oc = OracleKVCache(B, ca.capacity, n_kv, d)
    if prefix:
        oc.append(pk.astype(np.float64), pv.astype(np.float64))
    wa, wb = sa.decode_workspace(ca, n_q), sa.decode_workspace(cb, n_q)
    qra = torch.empty((B, 1, n_q, d), dtype=torch.bfloat16, device="cuda")
    qrb = torch.empty_like(qra)
    err = 0.0
    for s in range(steps):
        q, k, v = _draw((B, 1, n_q, d), rng), _draw((B, 1, n_kv, d), rng), _draw((B, 1, n_kv, d), rng)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        ca.append_rope_qk(qd, kd, vd, ly, q_out=qra)
        oa = sa.sinkattn_decode(qra, ca, s_t, W, sm, workspace=wa)
        ob = sa.sinkattn_decode_step(cb, qd, kd, vd, s_t, W, sm, ly, q_rot=qrb, workspace=wb)
        torch.cuda.synchronize()
        assert ca.offset == cb.offset == prefix + s + 1
        assert torch.equal(_bits(oa), _bits(ob)), ("out", s)
        assert torch.equal(_bits(qra), _bits(qrb)), ("q_rot", s)
        want, _, _ = decode_step(oc, q, k, v, sinks, W, sm, inv, conc, "bf16")
        err = max(err, max_abs(host(ob), want))
    # the rows the fused step wrote, and everything else in the buffers
    assert torch.equal(_bits(ca.k), _bits(cb.k))
    assert torch.equal(_bits(ca.v), _bits(cb.v))
    assert err <= TOL["bf16"], err


def test_decode_step_without_q_rot_and_unchanged_inputs():
    """q_rot=None writes no rotated Q; the raw q, k, v are left as they were."""
    rng = np.random.default_rng(5)
    B, n_q, n_kv, d = 2, 16, 2, 64
    y = Yarn()
    ly = lib_yarn(d, y)
    s_t = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    (ca, cb), _, _ = _caches(B, 90, 3, n_kv, d, rng)
    for _ in range(3):
        q, k, v = _draw((B, 1, n_q, d), rng), _draw((B, 1, n_kv, d), rng), _draw((B, 1, n_kv, d), rng)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        keep = [t.clone() for t in (qd, kd, vd)]
        qr = ca.append_rope_qk(qd, kd, vd, ly)
        oa = sa.sinkattn_decode(qr, ca, s_t, 0, 0.125)
        ob = sa.sinkattn_decode_step(cb, qd, kd, vd, s_t, 0, 0.125, ly)
        torch.cuda.synchronize()
        assert torch.equal(_bits(oa), _bits(ob))
        for a, b in zip(keep, (qd, kd, vd)):
            assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("W,prefix,d,n_q,n_kv", [(128, 100, 64, 16, 2), (64, 0, 64, 16, 2),
                                                  (64, 40, 96, 8, 4), (96, 200, 128, 16, 1)])
def test_decode_step_on_a_ring(W, prefix, d, n_q, n_kv):
    """A ring cache: the token's slot is p mod W, anywhere in the ring once it
    has wrapped; bit-equal to append_rope_qk + decode on a second ring, and
    within tolerance of the oracle's ring."""
    rng = np.random.default_rng(W + prefix + d)
    B, steps = 2, 3 * W // 2 + 5
    y = Yarn()
    ly = lib_yarn(d, y)
    sm = 1.0 / np.sqrt(d)
    sinks = rng.standard_normal(n_q).astype(np.float32)
    s_t = torch.from_numpy(sinks).cuda()
    ra = sa.KVRing.empty(B, W, n_kv, d, fill=float("nan"))
    rb = sa.KVRing.empty(B, W, n_kv, d, fill=float("nan"))
    oring = OracleRingCache(B, W, n_kv, d)
    if prefix:
        pk, pv = _draw((B, prefix, n_kv, d), rng), _draw((B, prefix, n_kv, d), rng)
        for r in (ra, rb):
            r.append(dev(pk, "bf16"), dev(pv, "bf16"))
        oring.append(pk.astype(np.float64), pv.astype(np.float64))
    wa, wb = sa.decode_workspace(ra, n_q), sa.decode_workspace(rb, n_q)
    qra = torch.empty((B, 1, n_q, d), dtype=torch.bfloat16, device="cuda")
    qrb = torch.empty_like(qra)
    err = 0.0
    for s in range(steps):
        q, k, v = _draw((B, 1, n_q, d), rng), _draw((B, 1, n_kv, d), rng), _draw((B, 1, n_kv, d), rng)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        ra.append_rope_qk(qd, kd, vd, ly, q_out=qra)
        oa = sa.sinkattn_decode(qra, ra, s_t, W, sm, workspace=wa)
        ob = sa.sinkattn_decode_step(rb, qd, kd, vd, s_t, W, sm, ly, q_rot=qrb, workspace=wb)
        torch.cuda.synchronize()
        assert torch.equal(_bits(oa), _bits(ob)), s
        assert torch.equal(_bits(qra), _bits(qrb)), s
        p = oring.offset
        oring.append(oracle_rot(k, p, d, y, "bf16"), v.astype(np.float64))
        want = ring_decode(oring, oracle_rot(q, p, d, y, "bf16"), sinks, sm)
        err = max(err, max_abs(host(ob), want))
    assert ra.offset == rb.offset == prefix + steps
    assert torch.equal(_bits(ra.k), _bits(rb.k)) and torch.equal(_bits(ra.v), _bits(rb.v))
    assert err <= TOL["bf16"], err


def test_decode_step_fills_the_cache_to_capacity():
    """Steps up to the last row of the cache (row C - 1, the last slot of its
    32-row block), then a step past it is refused with nothing written."""
    rng = np.random.default_rng(11)
    B, n_q, n_kv, d = 1, 8, 2, 64
    y = Yarn()
    ly = lib_yarn(d, y)
    s_t = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    C = 64
    (ca, cb), _, _ = _caches(B, C - 3, 3, n_kv, d, rng, C=C)
    assert ca.capacity == cb.capacity == C
    for _ in range(3):
        q, k, v = _draw((B, 1, n_q, d), rng), _draw((B, 1, n_kv, d), rng), _draw((B, 1, n_kv, d), rng)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        qr = ca.append_rope_qk(qd, kd, vd, ly)
        oa = sa.sinkattn_decode(qr, ca, s_t, 0, 0.125)
        ob = sa.sinkattn_decode_step(cb, qd, kd, vd, s_t, 0, 0.125, ly)
        torch.cuda.synchronize()
        assert torch.equal(_bits(oa), _bits(ob))
    assert cb.offset == C
    k_before, v_before = cb.k.clone(), cb.v.clone()
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_decode_step(cb, qd, kd, vd, s_t, 0, 0.125, ly)
    torch.cuda.synchronize()
    assert cb.offset == C
    assert torch.equal(_bits(cb.k), _bits(k_before)) and torch.equal(_bits(cb.v), _bits(v_before))
    assert torch.equal(_bits(ca.k), _bits(cb.k)) and torch.equal(_bits(ca.v), _bits(cb.v))


def _random_case(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 96, 128]))
    n_kv = int(r.choice([1, 2, 4, 8]))
    q_mult = int(r.choice([1, 2, 3, 4, 6, 8, 16]))
    B = int(r.integers(1, 4))
    W = int(r.choice([0, 0, 17, 128, 300]))
    prefix = int(r.integers(0, 3000))
    steps = int(r.integers(1, 5))
    return B, prefix, steps, q_mult * n_kv, n_kv, d, W


@pytest.mark.parametrize("seed", range(12))
def test_decode_step_random_shapes(seed):
    """Seeded random shapes (head dimension, group size, batch, band width,
    cache fill): the fused step stays bit-equal to the separate calls."""
    B, prefix, steps, n_q, n_kv, d, W = _random_case(seed)
    rng = np.random.default_rng(seed + 100)
    y = Yarn()
    ly = lib_yarn(d, y)
    sm = 1.0 / np.sqrt(d)
    s_t = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    (ca, cb), _, _ = _caches(B, prefix, steps, n_kv, d, rng)
    wa, wb = sa.decode_workspace(ca, n_q), sa.decode_workspace(cb, n_q)
    qra = torch.empty((B, 1, n_q, d), dtype=torch.bfloat16, device="cuda")
    qrb = torch.empty_like(qra)
    for s in range(steps):
        q, k, v = _draw((B, 1, n_q, d), rng), _draw((B, 1, n_kv, d), rng), _draw((B, 1, n_kv, d), rng)
        qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
        ca.append_rope_qk(qd, kd, vd, ly, q_out=qra)
        oa = sa.sinkattn_decode(qra, ca, s_t, W, sm, workspace=wa)
        ob = sa.sinkattn_decode_step(cb, qd, kd, vd, s_t, W, sm, ly, q_rot=qrb, workspace=wb)
        torch.cuda.synchronize()
        assert torch.equal(_bits(oa), _bits(ob)), (seed, s)
        assert torch.equal(_bits(qra), _bits(qrb)), (seed, s)
    assert torch.equal(_bits(ca.k), _bits(cb.k)) and torch.equal(_bits(ca.v), _bits(cb.v))
