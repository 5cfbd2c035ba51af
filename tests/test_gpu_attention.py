"""GPU parity of sinkattn_prefill / sinkattn_decode against the fp64 oracle
at sizes the oracle finishes in seconds, spanning several 64-key tiles with
ragged tails, offsets that do not align to tiles, every supported head
dimension, q_mult in {1, 2, 3, 4, 8, 16}, sinks finite and -inf, full causal
and band layers.  Tolerance: max-abs 2e-2 (bf16 I/O, fp32 accumulate) and
1e-5 (fp32 I/O).  Mask edges are checked exactly with probe keys.
"""
import numpy as np
import pytest
import torch

from oracle.attention import sink_attention
from oracle.kvcache import OracleKVCache
from oracle.layer import decode_step, prefill_layer
from workloads import Yarn, bf16_round
from tests.gpu_helpers import (TOL, TORCH_DT, dev, gpu_prefill_layer, host, lib_yarn,
                               max_abs, oracle_tables)

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _draw(shape, rng, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


PREFILL_CASES = [
    # B, prefix, T, n_q, n_kv, d, window, sink_inf, dtype
    (2, 0, 333, 8, 2, 64, 0, False, "bf16"),
    (2, 0, 333, 8, 2, 64, 128, False, "bf16"),
    (1, 37, 200, 8, 4, 96, 128, False, "bf16"),
    (1, 100, 150, 16, 2, 128, 17, False, "bf16"),
    (1, 0, 257, 64, 8, 64, 128, True, "bf16"),
    (1, 64, 129, 64, 8, 64, 0, False, "bf16"),
    (2, 5, 65, 4, 4, 64, 0, False, "bf16"),            # q_mult 1
    (1, 3, 100, 6, 2, 64, 40, False, "bf16"),          # q_mult 3
    (1, 0, 1, 8, 2, 96, 0, False, "bf16"),             # a single query
    (1, 1000, 31, 16, 1, 64, 0, True, "bf16"),         # q_mult 16, long prefix
    (1, 0, 128, 8, 2, 64, 0, False, "f32"),            # the tiny fp32 layers
    (1, 0, 128, 8, 2, 64, 32, False, "f32"),
    (2, 19, 77, 6, 3, 40, 9, True, "f32"),
    (1, 50, 140, 8, 2, 96, 0, True, "bf16"),           # no sink on the v_dot2-sum shapes
    (1, 0, 100, 16, 2, 128, 64, True, "bf16"),
    (1, 70, 190, 16, 2, 64, 0, "mixed", "bf16"),       # every other head without a sink
    (1, 2023, 300, 16, 2, 64, 1000, False, "bf16"),    # a band wider than the band shape takes
    (1, 2000, 300, 16, 2, 64, 1000, False, "bf16"),    #   the full-causal walk (in threes; first unit skipped)
    (1, 30, 160, 8, 2, 96, 48, "mixed", "bf16"),
]


@pytest.mark.parametrize("B,prefix,T,n_q,n_kv,d,W,sink_inf,dtype", PREFILL_CASES)
def test_prefill_matches_oracle(B, prefix, T, n_q, n_kv, d, W, sink_inf, dtype):
    rng = np.random.default_rng(T * 7 + d + prefix)
    y = Yarn()
    sm = 1.0 / np.sqrt(d)
    C = ((prefix + T + 31) // 32) * 32 + 32
    q = _draw((B, T, n_q, d), rng, dtype)
    k = _draw((B, T, n_kv, d), rng, dtype)
    v = _draw((B, T, n_kv, d), rng, dtype)
    sinks = np.full(n_q, -np.inf, np.float32) if sink_inf is True else rng.standard_normal(n_q).astype(np.float32)
    if sink_inf == "mixed":
        sinks[::2] = -np.inf
    pk = _draw((B, prefix, n_kv, d), rng, dtype)
    pv = _draw((B, prefix, n_kv, d), rng, dtype)

    cache = sa.KVCache.empty(B, C, n_kv, d, dtype=TORCH_DT[dtype], fill=float("nan"))
    if prefix:
        cache.append(dev(pk, dtype), dev(pv, dtype))
    s_t = torch.from_numpy(sinks).cuda()
    out, _, _ = gpu_prefill_layer(cache, q, k, v, s_t, W, sm, y, dtype)
    torch.cuda.synchronize()
    got = host(out)

    inv, c = oracle_tables(d, y)
    oc = OracleKVCache(B, C, n_kv, d)
    if prefix:
        oc.append(pk.astype(np.float64), pv.astype(np.float64))
    want, _, _ = prefill_layer(oc, q, k, v, sinks, W, sm, inv, c, dtype)
    assert np.all(np.isfinite(got))
    err = max_abs(got, want)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("W", [0, 128])
@pytest.mark.parametrize("offset", [0, 64, 65536 - 40])
def test_mask_edges_exact(W, offset):
    """A probe key j with a +30 logit and a one-hot value: the output's probe
    coordinate is ~1 iff j is allowed for the query, and exactly 0 if not."""
    B, n_q, n_kv, d, T = 1, 8, 1, 64, 200
    C = ((offset + T + 31) // 32) * 32
    cache = sa.KVCache.empty(B, C, n_kv, d, fill=0.0)
    if offset:
        z = torch.zeros((B, offset, n_kv, d), dtype=torch.bfloat16, device="cuda")
        cache.append(z, z)
    q = torch.zeros((B, T, n_q, d), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = 1.0
    k = torch.zeros((B, T, n_kv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((B, T, n_kv, d), dtype=torch.bfloat16, device="cuda")
    cache.append(k, v)
    sinks = torch.full((n_q,), -float("inf"), device="cuda")
    probes = []
    for t in (0, 1, 63, 64, 127, 128, 129, 199):
        p = offset + t
        for j in (p, p + 1, p - W + 1, p - W):
            if 0 <= j < offset + T:
                probes.append((t, p, j))
    for (t, p, j) in probes:
        cache.k[0, j, 0, 0] = 30.0
        cache.v[0, j // 32, 0, 1, j % 32] = 1.0          # V[j][1] in the blocked layout
        out = sa.sinkattn_prefill(q[:, t:t + 1].contiguous(), cache, sinks, W, 1.0, p)
        torch.cuda.synchronize()
        val = float(out[0, 0, 0, 1])
        allowed = j <= p and (W == 0 or j > p - W)
        if allowed:
            assert val > 0.99, (t, p, j)
        else:
            assert val == 0.0, (t, p, j)
        cache.k[0, j, 0, 0] = 0.0
        cache.v[0, j // 32, 0, 1, j % 32] = 0.0


DECODE_CASES = [
    # B, prefix, steps, n_q, n_kv, d, window, dtype, sink_inf
    (2, 1000, 6, 64, 8, 64, 0, "bf16", False),
    (2, 1000, 6, 64, 8, 64, 128, "bf16", False),
    (1, 300, 4, 8, 4, 96, 0, "bf16", False),
    (3, 77, 5, 16, 1, 128, 50, "bf16", False),
    (1, 5000, 3, 32, 8, 64, 0, "bf16", False),
    (1, 2000, 3, 16, 4, 64, 512, "bf16", False),       # band wider than one split: lo inside a split
    (2, 1000, 3, 64, 8, 64, 0, "bf16", True),          # no sink, split span + merge
    (2, 1000, 3, 64, 8, 64, 128, "bf16", True),        # no sink, single-split span
    (1, 150, 3, 8, 2, 96, 0, "bf16", True),            # no sink, whole cache in one split
    (1, 320, 12, 8, 2, 64, 0, "bf16", False),          # folded splits: 12 pieces over 11 blocks, one empty
    (1, 5000, 2, 32, 8, 64, 0, "bf16", True),          # no sink, folded splits
    (1, 600, 3, 16, 2, 64, 256, "bf16", False),        # 256-row band: nine blocks, one wave walks three
    (2, 250, 10, 16, 4, 64, 0, "bf16", True),          # full layer across 256 rows: short, then split
    (1, 120, 4, 8, 2, 64, 0, "f32", False),
    (1, 120, 4, 8, 2, 64, 32, "f32", False),
    (1, 300, 2, 8, 2, 64, 0, "f32", True),
]


def _decode_sweep(B, prefix, steps, n_q, n_kv, d, W, dtype, sinks, pk, pv, rng, kscale=None):
    """Append the prefix, then run `steps` decode steps on the GPU and in the
    oracle; returns the max-abs difference of each step."""
    y = Yarn()
    sm = 1.0 / np.sqrt(d)
    C = ((prefix + steps + 31) // 32) * 32 + 32
    s_t = torch.from_numpy(sinks).cuda()
    cache = sa.KVCache.empty(B, C, n_kv, d, dtype=TORCH_DT[dtype], fill=float("nan"))
    cache.append(dev(pk, dtype), dev(pv, dtype))
    ws = sa.decode_workspace(cache, n_q)
    inv, c = oracle_tables(d, y)
    oc = OracleKVCache(B, C, n_kv, d)
    oc.append(pk.astype(np.float64), pv.astype(np.float64))
    ly = lib_yarn(d, y)
    errs = []
    for s in range(steps):
        q = _draw((B, 1, n_q, d), rng, dtype)
        k = _draw((B, 1, n_kv, d), rng, dtype)
        if kscale is not None:
            k = (bf16_round if dtype == "bf16" else np.float32)(k * kscale)
        v = _draw((B, 1, n_kv, d), rng, dtype)
        o = cache.offset
        qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
        sa.yarn_rope_apply(qd, o, ly)
        sa.yarn_rope_apply(kd, o, ly)
        cache.append(kd, vd)
        out = sa.sinkattn_decode(qd, cache, s_t, W, sm, workspace=ws)
        torch.cuda.synchronize()
        want, _, _ = decode_step(oc, q, k, v, sinks, W, sm, inv, c, dtype)
        got = host(out)
        assert np.all(np.isfinite(got)), s
        errs.append(max_abs(got, want))
    return errs


@pytest.mark.parametrize("B,prefix,steps,n_q,n_kv,d,W,dtype,sink_inf", DECODE_CASES)
def test_decode_matches_oracle(B, prefix, steps, n_q, n_kv, d, W, dtype, sink_inf):
    rng = np.random.default_rng(prefix + d + steps + 7 * sink_inf)
    sinks = (np.full(n_q, -np.inf, np.float32) if sink_inf
             else rng.standard_normal(n_q).astype(np.float32))
    pk = _draw((B, prefix, n_kv, d), rng, dtype)
    pv = _draw((B, prefix, n_kv, d), rng, dtype)
    errs = _decode_sweep(B, prefix, steps, n_q, n_kv, d, W, dtype, sinks, pk, pv, rng)
    assert max(errs) <= TOL[dtype], errs


@pytest.mark.parametrize("W,sink_inf", [(0, False), (0, True), (128, False)])
def test_decode_growing_logits(W, sink_inf):
    """Keys whose size grows 20-fold along the cache: the scores of later
    key blocks pass the running max by far more than the lazy slack (2^8 in
    probability), many times within one split, so the kernel's rescale runs
    mid-span; the largest scaled logits reach ~100 (e^100 would overflow an
    unscaled fp32 sum)."""
    B, prefix, steps, n_q, n_kv, d = 1, 2400, 2, 16, 2, 64
    rng = np.random.default_rng(31 + W)
    growth = (1.0 + 19.0 * np.arange(prefix) / prefix).astype(np.float32)[None, :, None, None]
    pk = bf16_round(_draw((B, prefix, n_kv, d), rng, "bf16") * growth)
    pv = _draw((B, prefix, n_kv, d), rng, "bf16")
    sinks = (np.full(n_q, -np.inf, np.float32) if sink_inf
             else rng.standard_normal(n_q).astype(np.float32))
    errs = _decode_sweep(B, prefix, steps, n_q, n_kv, d, W, "bf16", sinks, pk, pv, rng,
                         kscale=20.0)
    assert max(errs) <= TOL["bf16"], errs


@pytest.mark.parametrize("W", [0, 128, 512])
@pytest.mark.parametrize("n_rows", [201, 1000, 65536])
def test_decode_mask_edges_exact(W, n_rows):
    """Decode's band and causal edges, bit-exact: the query sits at p = n_rows-1
    (its own row just appended); a probe key j gets a +30 logit and a one-hot
    value.  The probe coordinate of the output is ~1 iff j is allowed
    (p-W < j <= p) and exactly 0 otherwise; rows past p hold NaN and must
    not leak.  201 rows run as one split, 1000 and 65536 through split
    partials and the merge (W = 512 with its lower edge inside a split)."""
    B, n_q, n_kv, d = 1, 8, 1, 64
    C = ((n_rows + 31) // 32) * 32 + 64
    cache = sa.KVCache.empty(B, C, n_kv, d, fill=float("nan"))
    z = torch.zeros((B, n_rows, n_kv, d), dtype=torch.bfloat16, device="cuda")
    cache.append(z, z)
    p = n_rows - 1
    q = torch.zeros((B, 1, n_q, d), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = 1.0
    sinks = torch.full((n_q,), -float("inf"), device="cuda")
    ws = sa.decode_workspace(cache, n_q)
    for j in (p, p - 1, p - W + 1, p - W, 0):
        if j < 0 or (W == 0 and j in (p - W + 1, p - W)):
            continue
        cache.k[0, j, 0, 0] = 30.0
        cache.v[0, j // 32, 0, 1, j % 32] = 1.0           # V[j][1] in the blocked layout
        out = sa.sinkattn_decode(q, cache, sinks, W, 1.0, workspace=ws)
        torch.cuda.synchronize()
        o = out[0, 0].float().cpu().numpy()
        assert np.all(np.isfinite(o)), (p, j)
        allowed = j <= p and (W == 0 or j > p - W)
        if allowed:
            assert np.all(o[:, 1] > 0.99), (W, p, j, o[:, 1])
        else:
            assert np.all(o[:, 1] == 0.0), (W, p, j, o[:, 1])
        cache.k[0, j, 0, 0] = 0.0
        cache.v[0, j // 32, 0, 1, j % 32] = 0.0


@pytest.mark.parametrize("W", [0, 7])
def test_decode_steps_equal_prefill_on_gpu(W):
    """Token-by-token decode reproduces one prefill of the same tokens: both
    within tolerance of the oracle, and the two caches bit-identical."""
    B, T, n_q, n_kv, d = 1, 70, 16, 2, 64
    rng = np.random.default_rng(5)
    y = Yarn()
    q = _draw((B, T, n_q, d), rng, "bf16")
    k = _draw((B, T, n_kv, d), rng, "bf16")
    v = _draw((B, T, n_kv, d), rng, "bf16")
    sinks = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    c1 = sa.KVCache.empty(B, 96, n_kv, d, fill=float("nan"))
    full, _, _ = gpu_prefill_layer(c1, q, k, v, sinks, W, 0.125, y, "bf16")
    c2 = sa.KVCache.empty(B, 96, n_kv, d, fill=float("nan"))
    ly = lib_yarn(d, y)
    outs = []
    for t in range(T):
        qd, kd, vd = dev(q[:, t:t + 1], "bf16"), dev(k[:, t:t + 1], "bf16"), dev(v[:, t:t + 1], "bf16")
        o = c2.offset
        sa.yarn_rope_apply(qd, o, ly)
        sa.yarn_rope_apply(kd, o, ly)
        c2.append(kd, vd)
        outs.append(sa.sinkattn_decode(qd, c2, sinks, W, 0.125))
        assert c2.offset == t + 1
    torch.cuda.synchronize()
    dec = host(torch.cat(outs, 1))
    assert max_abs(dec, host(full)) <= 2e-2
    assert torch.equal(c1.k[:, :T].view(torch.int16), c2.k[:, :T].view(torch.int16))
    assert torch.equal(c1.v_rows()[:, :T].view(torch.int16), c2.v_rows()[:, :T].view(torch.int16))


def test_decode_is_deterministic_across_restore():
    """Sweep A, restore, sweep B, restore, sweep A again: A == A bit for bit."""
    B, n_q, n_kv, d, prefix = 2, 64, 8, 64, 3000
    rng = np.random.default_rng(9)
    cache = sa.KVCache.empty(B, 3072 + 64, n_kv, d, fill=float("nan"))
    cache.append(dev(_draw((B, prefix, n_kv, d), rng, "bf16"), "bf16"),
                 dev(_draw((B, prefix, n_kv, d), rng, "bf16"), "bf16"))
    sinks = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    snap = cache.snapshot()
    ly = lib_yarn(d, Yarn())

    def sweep(seed):
        r = np.random.default_rng(seed)
        outs = []
        for _ in range(8):
            qd = dev(_draw((B, 1, n_q, d), r, "bf16"), "bf16")
            kd = dev(_draw((B, 1, n_kv, d), r, "bf16"), "bf16")
            vd = dev(_draw((B, 1, n_kv, d), r, "bf16"), "bf16")
            o = cache.offset
            sa.yarn_rope_apply(qd, o, ly)
            sa.yarn_rope_apply(kd, o, ly)
            cache.append(kd, vd)
            outs.append(sa.sinkattn_decode(qd, cache, sinks, 0, 0.125))
        torch.cuda.synchronize()
        return torch.cat(outs, 1).view(torch.int16).clone()

    a1 = sweep(0)
    cache.restore(snap)
    b = sweep(1)
    cache.restore(snap)
    a2 = sweep(0)
    assert torch.equal(a1, a2)
    assert not torch.equal(a1, b)


def test_prefill_is_deterministic():
    B, T, n_q, n_kv, d = 1, 300, 64, 8, 64
    rng = np.random.default_rng(11)
    cache = sa.KVCache.empty(B, 320, n_kv, d)
    cache.append(dev(_draw((B, T, n_kv, d), rng, "bf16"), "bf16"),
                 dev(_draw((B, T, n_kv, d), rng, "bf16"), "bf16"))
    q = dev(_draw((B, T, n_q, d), rng, "bf16"), "bf16")
    sinks = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    a = sa.sinkattn_prefill(q, cache, sinks, 0, 0.125, 0)
    b = sa.sinkattn_prefill(q, cache, sinks, 0, 0.125, 0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("scale_qk,growing", [(12.0, True), (12.0, False), (0.02, False)])
@pytest.mark.parametrize("sink_inf", [False, True])
def test_prefill_extreme_logits(scale_qk, growing, sink_inf):
    """Scores far from the sink: large logits that grow along the sequence
    (the reference must move several times mid-sequence), large logits from
    the start, and near-zero logits; with and without a sink."""
    B, T, n_q, n_kv, d = 1, 300, 8, 2, 64
    rng = np.random.default_rng(21)
    q = bf16_round((rng.standard_normal((B, T, n_q, d)) * scale_qk).astype(np.float32))
    k = rng.standard_normal((B, T, n_kv, d)).astype(np.float32) * scale_qk
    if growing:                       # key norms rise with position: later keys dominate
        k *= np.linspace(0.2, 1.0, T, dtype=np.float32)[None, :, None, None]
    k = bf16_round(k)
    v = bf16_round(rng.standard_normal((B, T, n_kv, d)).astype(np.float32))
    sinks = np.full(n_q, -np.inf, np.float32) if sink_inf else rng.standard_normal(n_q).astype(np.float32)
    cache = sa.KVCache.empty(B, 320, n_kv, d, fill=float("nan"))
    cache.append(dev(k, "bf16"), dev(v, "bf16"))          # K taken as already rotated
    out = sa.sinkattn_prefill(dev(q, "bf16"), cache, torch.from_numpy(sinks).cuda(), 0, 0.125, 0)
    torch.cuda.synchronize()
    got = host(out)
    want = sink_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                          sinks, 0, 0, 0.125)
    assert np.all(np.isfinite(got))
    assert max_abs(got, want) <= 2e-2, max_abs(got, want)


ROPE_PREFILL_CASES = [
    # B, prefix, T, n_q, n_kv, d, window
    (2, 0, 333, 8, 2, 64, 0),
    (1, 37, 200, 8, 4, 96, 128),
    (1, 100, 150, 16, 2, 128, 17),
    (1, 64, 129, 64, 8, 64, 0),
    (1, 5, 300, 4, 4, 128, 0),        # q_mult 1 at d = 128: the rotation table takes chunks
    (2, 7, 65, 8, 8, 96, 0),          # q_mult 1 at d = 96
    (1, 1000, 31, 16, 1, 64, 0),
]


@pytest.mark.parametrize("B,prefix,T,n_q,n_kv,d,W", ROPE_PREFILL_CASES)
def test_prefill_rope_equals_rope_then_prefill(B, prefix, T, n_q, n_kv, d, W):
    """sinkattn_prefill_rope on raw queries gives the bits of yarn_rope_apply
    followed by sinkattn_prefill."""
    rng = np.random.default_rng(T * 5 + d + prefix)
    ly = lib_yarn(d, Yarn())
    C = ((prefix + T + 31) // 32) * 32 + 32
    k = _draw((B, prefix + T, n_kv, d), rng, "bf16")
    v = _draw((B, prefix + T, n_kv, d), rng, "bf16")
    q = _draw((B, T, n_q, d), rng, "bf16")
    sinks = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    cache = sa.KVCache.empty(B, C, n_kv, d, fill=float("nan"))
    cache.append_rope(dev(k, "bf16"), dev(v, "bf16"), ly)
    q_raw = dev(q, "bf16")
    q_rot = torch.empty_like(q_raw)
    sa.yarn_rope_apply(q_raw, prefix, ly, out=q_rot)
    want = sa.sinkattn_prefill(q_rot, cache, sinks, W, 1.0 / np.sqrt(d), prefix)
    got = sa.sinkattn_prefill_rope(q_raw, cache, sinks, W, 1.0 / np.sqrt(d), prefix, ly)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert torch.equal(q_raw.view(torch.int16), dev(q, "bf16").view(torch.int16))  # q untouched


def test_prefill_rope_matches_oracle():
    """The fused path against the fp64 oracle layer (rotation included)."""
    B, T, n_q, n_kv, d, W = 1, 200, 8, 4, 96, 128
    rng = np.random.default_rng(11)
    y = Yarn()
    ly = lib_yarn(d, y)
    q = _draw((B, T, n_q, d), rng, "bf16")
    k = _draw((B, T, n_kv, d), rng, "bf16")
    v = _draw((B, T, n_kv, d), rng, "bf16")
    sinks = rng.standard_normal(n_q).astype(np.float32)
    sm = 1.0 / np.sqrt(d)
    cache = sa.KVCache.empty(B, 256, n_kv, d, fill=float("nan"))
    cache.append_rope(dev(k, "bf16"), dev(v, "bf16"), ly)
    got = sa.sinkattn_prefill_rope(dev(q, "bf16"), cache, torch.from_numpy(sinks).cuda(), W, sm,
                                   0, ly)
    inv, conc = oracle_tables(d, y)
    want, _, _ = prefill_layer(OracleKVCache(B, 256, n_kv, d), q, k, v, sinks, W, sm, inv, conc,
                               "bf16")
    assert max_abs(host(got), want) <= TOL["bf16"]
