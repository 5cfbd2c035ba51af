"""GPU parity of the band layers' ring cache (kv_ring_create, kv_ring_stage,
kv_ring_commit, kv_ring_save / kv_ring_load, appends and decode on a ring)
against the oracle's ring (oracle/ring.py), at sizes the oracle finishes in
seconds: chunks shorter and longer than the window, offsets that do not
align to 32-row blocks, appends that wrap past the ring's end, decode sweeps
that overwrite every slot several times.  Outputs within 2e-2 (bf16) / 1e-5
(fp32) of the oracle; V rows bit-exact; rotated K and Q rows within one unit
in the last place of the oracle's and bit-equal to the library's yarn_rope.
"""
import numpy as np
import pytest
import torch

from oracle.ring import OracleRingCache, ring_decode, ring_prefill
from workloads import Yarn, bf16_round
from tests.gpu_helpers import TOL, TORCH_DT, dev, host, lib_yarn, max_abs, oracle_rot

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _draw(shape, rng, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def _ulps(got_f64, want_f64, dtype):
    """Distance in units of the last place between two arrays of values that
    are exact in `dtype` (NaN where either is NaN)."""
    if dtype == "bf16":
        a = torch.from_numpy(np.ascontiguousarray(got_f64)).to(torch.bfloat16).view(torch.int16)
        b = torch.from_numpy(np.ascontiguousarray(want_f64)).to(torch.bfloat16).view(torch.int16)
    else:
        a = torch.from_numpy(np.ascontiguousarray(got_f64, np.float32)).view(torch.int32)
        b = torch.from_numpy(np.ascontiguousarray(want_f64, np.float32)).view(torch.int32)
    return np.abs(a.numpy().astype(np.int64) - b.numpy().astype(np.int64))


def _stage_rows(W, chunk):
    return ((W - 1 + chunk + 31) // 32) * 32


def _check_ring_rows(ring, oring, dtype, k_exact=False):
    """Live slots of the device ring against the oracle ring's: V bit for
    bit; K (rotated on both sides, each with its own sin/cos) within one
    unit in the last place, or bit for bit when it was copied unrotated."""
    torch.cuda.synchronize()
    pos, live = oring.live()
    Kd = host(ring.k)[:, live]
    Vd = host(ring.v_rows())[:, live]
    assert np.array_equal(Vd, oring.V[:, live])
    if k_exact:
        assert np.array_equal(Kd, oring.K[:, live])
    else:
        assert _ulps(Kd, oring.K[:, live], dtype).max() <= 1


RING_CASES = [
    # B, n_q, n_kv, d, W, prefill chunks, decode steps, dtype
    (2, 8, 2, 64, 32, [45, 7, 64], 70, "bf16"),
    (1, 8, 4, 96, 128, [300, 129, 1], 140, "bf16"),
    (1, 16, 2, 128, 64, [64, 64], 66, "bf16"),
    (1, 64, 8, 64, 128, [257], 130, "bf16"),
    (2, 6, 3, 40, 32, [50, 33], 40, "f32"),
]


@pytest.mark.parametrize("B,n_q,n_kv,d,W,chunks,steps,dtype", RING_CASES)
def test_ring_layer_matches_oracle(B, n_q, n_kv, d, W, chunks, steps, dtype):
    rng = np.random.default_rng(W * 131 + d + len(chunks))
    y = Yarn()
    ly = lib_yarn(d, y)
    sm = 1.0 / np.sqrt(d)
    sinks = rng.standard_normal(n_q).astype(np.float32)
    s_t = torch.from_numpy(sinks).cuda()
    dt = TORCH_DT[dtype]
    ring = sa.KVRing.empty(B, W, n_kv, d, dtype=dt, fill=float("nan"))
    stage = sa.KVCache.empty(B, _stage_rows(W, max(chunks)), n_kv, d, dtype=dt,
                             fill=float("nan"))
    oring = OracleRingCache(B, W, n_kv, d)
    for T in chunks:
        o = ring.offset
        q, k, v = (_draw((B, T, n_q, d), rng, dtype), _draw((B, T, n_kv, d), rng, dtype),
                   _draw((B, T, n_kv, d), rng, dtype))
        ring.stage(stage)
        assert stage.offset == o and stage.base == max(0, o - (W - 1))
        q_rot = stage.append_rope_qk(dev(q, dtype), dev(k, dtype), dev(v, dtype), ly)
        out = sa.sinkattn_prefill(q_rot, stage, s_t, W, sm, o)
        ring.commit(stage)
        assert ring.offset == o + T
        q_ref = oracle_rot(q, o, d, y, dtype)
        k_ref = oracle_rot(k, o, d, y, dtype)
        want = ring_prefill(oring, q_ref, k_ref, v.astype(np.float64), sinks, sm)
        torch.cuda.synchronize()
        assert _ulps(host(q_rot), q_ref, dtype).max() <= 1
        got = host(out)
        assert np.all(np.isfinite(got))
        assert max_abs(got, want) <= TOL[dtype], ("prefill", T, max_abs(got, want))
        _check_ring_rows(ring, oring, dtype)
    ws = sa.decode_workspace(ring, n_q)
    err = 0.0
    for s in range(steps):
        p = ring.offset
        q, k, v = (_draw((B, 1, n_q, d), rng, dtype), _draw((B, 1, n_kv, d), rng, dtype),
                   _draw((B, 1, n_kv, d), rng, dtype))
        q_rot = ring.append_rope_qk(dev(q, dtype), dev(k, dtype), dev(v, dtype), ly)
        out = sa.sinkattn_decode(q_rot, ring, s_t, W, sm, workspace=ws)
        oring.append(oracle_rot(k, p, d, y, dtype), v.astype(np.float64))
        want = ring_decode(oring, oracle_rot(q, p, d, y, dtype), sinks, sm)
        err = max(err, max_abs(host(out), want))
    assert err <= TOL[dtype], ("decode", err)
    assert ring.base == max(0, ring.offset - W)
    _check_ring_rows(ring, oring, dtype)


def test_ring_decode_from_empty_ring():
    """Decode from position 0: the ring fills row by row (rows past the last
    position hold NaN and must not be read), then wraps."""
    B, n_q, n_kv, d, W = 2, 8, 2, 64, 32
    rng = np.random.default_rng(11)
    y = Yarn()
    ly = lib_yarn(d, y)
    sinks = rng.standard_normal(n_q).astype(np.float32)
    s_t = torch.from_numpy(sinks).cuda()
    ring = sa.KVRing.empty(B, W, n_kv, d, fill=float("nan"))
    oring = OracleRingCache(B, W, n_kv, d)
    ws = sa.decode_workspace(ring, n_q)
    for p in range(W + 9):
        q, k, v = (_draw((B, 1, n_q, d), rng, "bf16"), _draw((B, 1, n_kv, d), rng, "bf16"),
                   _draw((B, 1, n_kv, d), rng, "bf16"))
        q_rot = ring.append_rope_qk(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), ly)
        out = host(sa.sinkattn_decode(q_rot, ring, s_t, W, 0.125, workspace=ws))
        oring.append(oracle_rot(k, p, d, y, "bf16"), v.astype(np.float64))
        want = ring_decode(oring, oracle_rot(q, p, d, y, "bf16"), sinks, 0.125)
        assert np.all(np.isfinite(out))
        assert max_abs(out, want) <= TOL["bf16"], (p, max_abs(out, want))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_long_and_wrapping_appends(dtype):
    """Appends longer than the ring keep the last W rows; an append that
    crosses the ring's end is written in two runs; every query row of
    append_rope_qk is rotated even where its key row is not kept."""
    B, n_q, n_kv, d, W = 2, 4, 2, 64, 32
    rng = np.random.default_rng(5)
    y = Yarn()
    ly = lib_yarn(d, y)
    ring = sa.KVRing.empty(B, W, n_kv, d, dtype=TORCH_DT[dtype], fill=float("nan"))
    oring = OracleRingCache(B, W, n_kv, d)
    for T, rope in ((20, False), (50, True), (2 * W + 37, True), (13, False), (W, True)):
        p = ring.offset
        k, v = _draw((B, T, n_kv, d), rng, dtype), _draw((B, T, n_kv, d), rng, dtype)
        if rope:
            q = _draw((B, T, n_q, d), rng, dtype)
            q_rot = ring.append_rope_qk(dev(q, dtype), dev(k, dtype), dev(v, dtype), ly)
            torch.cuda.synchronize()
            assert _ulps(host(q_rot), oracle_rot(q, p, d, y, dtype), dtype).max() <= 1, T
            oring.append(oracle_rot(k, p, d, y, dtype), v.astype(np.float64))
            # the kept K rows equal yarn_rope's (the library's own rotation) bit for bit
            kr = dev(k, dtype)
            sa.yarn_rope_apply(kr, p, ly)
            torch.cuda.synchronize()
        else:
            ring.append(dev(k, dtype), dev(v, dtype))
            oring.append(k.astype(np.float64), v.astype(np.float64))
            kr = dev(k, dtype)
        torch.cuda.synchronize()
        keep = min(T, W)
        got_k = host(ring.k)[:, [(p + t) % W for t in range(T - keep, T)]]
        assert np.array_equal(got_k, host(kr)[:, T - keep:]), T
        assert ring.offset == oring.offset
        _check_ring_rows(ring, oring, dtype)


def test_ring_save_load_prefill_once_decode_many():
    B, n_q, n_kv, d, W = 1, 16, 2, 96, 64
    rng = np.random.default_rng(9)
    y = Yarn()
    ly = lib_yarn(d, y)
    sinks = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    ring = sa.KVRing.empty(B, W, n_kv, d, fill=float("nan"))
    stage = sa.KVCache.empty(B, _stage_rows(W, 200), n_kv, d, fill=float("nan"))
    q, k, v = (_draw((B, 200, n_q, d), rng, "bf16"), _draw((B, 200, n_kv, d), rng, "bf16"),
               _draw((B, 200, n_kv, d), rng, "bf16"))
    ring.stage(stage)
    stage.append_rope_qk(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), ly)
    ring.commit(stage)
    saved = ring.save()
    snap = ring.snapshot()
    ws = sa.decode_workspace(ring, n_q)

    def sweep(seed):
        r = np.random.default_rng(seed)
        outs = []
        for _ in range(2 * W + 3):                  # overwrites every slot twice
            qq, kk, vv = (_draw((B, 1, n_q, d), r, "bf16"), _draw((B, 1, n_kv, d), r, "bf16"),
                          _draw((B, 1, n_kv, d), r, "bf16"))
            q_rot = ring.append_rope_qk(dev(qq, "bf16"), dev(kk, "bf16"), dev(vv, "bf16"), ly)
            outs.append(sa.sinkattn_decode(q_rot, ring, sinks, W, 0.1, workspace=ws)
                        .view(torch.int16).clone())
        torch.cuda.synchronize()
        return torch.stack(outs)

    a1 = sweep(1)
    with pytest.raises(sa.SinkAttnError):
        ring.restore(snap)                          # slots were overwritten: refused
    ring.load(saved)
    assert ring.offset == 200
    b = sweep(2)
    ring.load(saved)
    a2 = sweep(1)
    assert torch.equal(a1, a2)
    assert not torch.equal(a1, b)


def test_prefill_rope_on_a_stage_uses_global_positions():
    """sinkattn_prefill_rope on a stage cache (base > 0) rotates each query
    at its global position: bit-equal to yarn_rope + sinkattn_prefill."""
    B, n_q, n_kv, d, W = 1, 8, 4, 96, 128
    rng = np.random.default_rng(13)
    y = Yarn()
    ly = lib_yarn(d, y)
    sinks = torch.from_numpy(rng.standard_normal(n_q).astype(np.float32)).cuda()
    ring = sa.KVRing.empty(B, W, n_kv, d)
    stage = sa.KVCache.empty(B, _stage_rows(W, 300), n_kv, d)
    for T in (300, 150):
        o = ring.offset
        q, k, v = (_draw((B, T, n_q, d), rng, "bf16"), _draw((B, T, n_kv, d), rng, "bf16"),
                   _draw((B, T, n_kv, d), rng, "bf16"))
        ring.stage(stage)
        qd = dev(q, "bf16")
        q_rot = stage.append_rope_qk(qd, dev(k, "bf16"), dev(v, "bf16"), ly)
        a = sa.sinkattn_prefill(q_rot, stage, sinks, W, 0.1, o)
        b = sa.sinkattn_prefill_rope(qd, stage, sinks, W, 0.1, o, ly)
        ring.commit(stage)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (T, stage.base)
    assert stage.base > 0


def test_ring_errors_on_device():
    B, n_q, n_kv, d, W = 1, 4, 2, 64, 32
    rng = np.random.default_rng(2)
    y = Yarn()
    ly = lib_yarn(d, y)
    sinks = torch.zeros(n_q, dtype=torch.float32, device="cuda")
    ring = sa.KVRing.empty(B, W, n_kv, d)
    k = dev(_draw((B, 40, n_kv, d), rng, "bf16"), "bf16")
    ring.append_rope(k, k, ly)
    ws = sa.decode_workspace(ring, n_q)
    q = dev(_draw((B, 1, n_q, d), rng, "bf16"), "bf16")
    with pytest.raises(sa.SinkAttnError):          # a ring serves only its own width
        sa.sinkattn_decode(q, ring, sinks, 16, 0.1, workspace=ws)
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_decode(q, ring, sinks, 0, 0.1, workspace=ws)
    small = sa.KVCache.empty(B, 32, n_kv, d)
    ring.stage(small)                               # W - 1 = 31 rows fit in 32
    tiny_ring = sa.KVRing.empty(B, 64, n_kv, d)
    k64 = dev(_draw((B, 64, n_kv, d), rng, "bf16"), "bf16")
    tiny_ring.append(k64, k64)
    with pytest.raises(sa.SinkAttnError):           # 63 rows do not fit in 32
        tiny_ring.stage(small)
    stage = sa.KVCache.empty(B, 128, n_kv, d)
    ring.stage(stage)
    qc = dev(_draw((B, 10, n_q, d), rng, "bf16"), "bf16")
    kc = dev(_draw((B, 10, n_kv, d), rng, "bf16"), "bf16")
    stage.append_rope(kc, kc, ly)
    with pytest.raises(sa.SinkAttnError):           # full causal needs keys below the base
        sa.sinkattn_prefill(qc, stage, sinks, 0, 0.1, 40)
    with pytest.raises(sa.SinkAttnError):           # a wider band than the stage holds
        sa.sinkattn_prefill(qc, stage, sinks, 64, 0.1, 40)
    sa.sinkattn_prefill(qc, stage, sinks, W, 0.1, 40)
    ring.append_rope(kc[:, :1], kc[:, :1], ly)      # the ring moves on: commit refused
    with pytest.raises(sa.SinkAttnError):
        ring.commit(stage)
    torch.cuda.synchronize()
