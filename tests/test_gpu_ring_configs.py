"""GPU parity of the band layers' ring cache on the workloads at their full
sizes, in the launch configuration bench.py times for the ring:

  GPT-OSS-Lite band layer  4096-token prefill through a stage cache, the
                           whole layer against the oracle; then 64 decode
                           steps on the 128-row ring, every step checked
  long decode band layer   the 131071-row prefix appended to a 128-row ring
                           (only its last 128 rows are kept), 64 decode
                           steps, every step of every sequence checked; the
                           ring's rows against the prefix's last rows
  handover band layer      65536-row prefix into the ring, a 2048-token chunk
                           through the stage, save, 32 decode steps, load,
                           32 steps under another seed, load, first sweep
                           replayed bit for bit

Oracle side: the raw seeded draws (workloads.py), the oracle's own RoPE,
and the plain band attention over the linear history of positions.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle.attention import attend_query, sink_attention
from oracle.rounding import round_to
from oracle.yarn import rope_apply
from tests.gpu_helpers import TOL, dev, host, lib_yarn, max_abs, oracle_tables

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _rot(w, x, offset):
    inv, c = oracle_tables(w.d_h, w.yarn)
    return round_to(rope_apply(np.asarray(x, np.float64), offset, inv, c), w.dtype)


def _band_layer(w):
    return [i for i, W in enumerate(w.windows) if W > 0][0]


def _stage_rows(W, T):
    return ((W - 1 + T + 31) // 32) * 32


class RingLayer:
    """The library's band layer on a ring: prefill chunks through a stage."""

    def __init__(self, w, layer, stage_T):
        self.w, self.layer, self.W = w, layer, w.windows[layer]
        self.ring = sa.KVRing.empty(w.B, self.W, w.n_kv, w.d_h, fill=float("nan"))
        self.stage = sa.KVCache.empty(w.B, _stage_rows(self.W, stage_T), w.n_kv, w.d_h,
                                      fill=float("nan"))
        self.sinks_h = wl.sinks(w, layer)
        self.sinks = torch.from_numpy(self.sinks_h).cuda()
        self.ly = lib_yarn(w.d_h, w.yarn)
        self.ws = sa.decode_workspace(self.ring, w.n_q)

    def prefill(self, q, k, v):
        o = self.ring.offset
        self.ring.stage(self.stage)
        q_rot = self.stage.append_rope_qk(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), self.ly)
        out = sa.sinkattn_prefill(q_rot, self.stage, self.sinks, self.W, self.w.sm_scale, o)
        self.ring.commit(self.stage)
        return out

    def decode(self, tok):
        q_rot = self.ring.append_rope_qk(dev(tok["q"], "bf16"), dev(tok["k"], "bf16"),
                                         dev(tok["v"], "bf16"), self.ly)
        return sa.sinkattn_decode(q_rot, self.ring, self.sinks, self.W, self.w.sm_scale,
                                  workspace=self.ws)


@pytest.mark.timeout(300)
def test_lite_band_layer_through_ring():
    w = wl.LITE_PREFILL
    layer = _band_layer(w)
    L = RingLayer(w, layer, w.T)
    x = wl.prefill_inputs(w, layer)
    out = host(L.prefill(x["q"], x["k"], x["v"]))
    assert L.ring.offset == w.T and L.stage.base == 0
    q_rot, k_rot = _rot(w, x["q"], 0), _rot(w, x["k"], 0)
    want = sink_attention(q_rot, k_rot, x["v"], L.sinks_h, 0, L.W, w.sm_scale)
    assert np.all(np.isfinite(out))
    assert max_abs(out, want) <= TOL["bf16"], max_abs(out, want)
    # decode on the ring: history of positions [T - W, T + steps)
    steps, base = 64, w.T - L.W
    Kh = np.concatenate([k_rot[:, base:], np.zeros((w.B, steps, w.n_kv, w.d_h))], 1)
    Vh = np.concatenate([x["v"][:, base:], np.zeros((w.B, steps, w.n_kv, w.d_h))], 1)
    err = 0.0
    for s in range(steps):
        p = w.T + s
        tok = wl.decode_token(w, layer, s)
        got = host(L.decode(tok))
        Kh[:, p - base] = _rot(w, tok["k"], p)[:, 0]
        Vh[:, p - base] = tok["v"][:, 0]
        q_r = _rot(w, tok["q"], p)
        for b in range(w.B):
            o = attend_query(q_r[b, 0], Kh[b], Vh[b], L.sinks_h, p - base, L.W, w.sm_scale)
            err = max(err, max_abs(got[b, 0], o))
    assert err <= TOL["bf16"], err


@pytest.mark.timeout(600)
def test_long_decode_band_layer_on_ring():
    w = wl.LONG_DECODE
    layer = _band_layer(w)
    W = w.windows[layer]
    L = RingLayer(w, layer, 1)
    px = wl.prefix_inputs(w, layer)
    L.ring.append(dev(px["prefix_k"], "bf16"), dev(px["prefix_v"], "bf16"))   # K counts as rotated
    assert L.ring.offset == w.prefix and L.ring.base == w.prefix - W
    torch.cuda.synchronize()
    slots = [p % W for p in range(w.prefix - W, w.prefix)]
    assert np.array_equal(host(L.ring.k)[:, slots], px["prefix_k"][:, -W:].astype(np.float64))
    assert np.array_equal(host(L.ring.v_rows())[:, slots], px["prefix_v"][:, -W:].astype(np.float64))
    base = w.prefix - W
    Kh = np.concatenate([px["prefix_k"][:, -W:], np.zeros((w.B, w.decode_steps, w.n_kv, w.d_h),
                                                           np.float32)], 1).astype(np.float64)
    Vh = np.concatenate([px["prefix_v"][:, -W:], np.zeros_like(Kh[:, W:], np.float32)],
                        1).astype(np.float64)
    del px
    err = 0.0
    for s in range(w.decode_steps):
        p = w.prefix + s
        tok = wl.decode_token(w, layer, s)
        got = host(L.decode(tok))
        Kh[:, p - base] = _rot(w, tok["k"], p)[:, 0]
        Vh[:, p - base] = tok["v"][:, 0]
        q_r = _rot(w, tok["q"], p)
        for b in range(w.B):
            o = attend_query(q_r[b, 0], Kh[b], Vh[b], L.sinks_h, p - base, W, w.sm_scale)
            err = max(err, max_abs(got[b, 0], o))
    assert L.ring.offset == w.prefix + w.decode_steps
    assert err <= TOL["bf16"], err


@pytest.mark.timeout(600)
def test_handover_band_layer_on_ring():
    w = wl.HANDOVER
    layer = _band_layer(w)
    W = w.windows[layer]
    rng = np.random.default_rng(7)
    L = RingLayer(w, layer, w.T)
    x = wl.prefill_inputs(w, layer)
    L.ring.append(dev(x["prefix_k"], "bf16"), dev(x["prefix_v"], "bf16"))
    out = host(L.prefill(x["q"], x["k"], x["v"]))
    assert L.stage.base == w.prefix - (W - 1)
    hb = w.prefix - W                                        # history starts here
    q_rot, k_rot = _rot(w, x["q"], w.prefix), _rot(w, x["k"], w.prefix)
    Kh = np.concatenate([x["prefix_k"][:, -W:], k_rot, np.zeros((1, 64, w.n_kv, w.d_h))], 1)
    Vh = np.concatenate([x["prefix_v"][:, -W:], x["v"], np.zeros((1, 64, w.n_kv, w.d_h))], 1)
    err = 0.0
    rows = sorted(set([0, 1, 126, 127, 128, 129, w.T - 1] + list(rng.choice(w.T, 24, False))))
    for t in rows:
        p = w.prefix + t
        o = attend_query(q_rot[0, t], Kh[0], Vh[0], L.sinks_h, p - hb, W, w.sm_scale)
        err = max(err, max_abs(out[0, t], o))
    assert err <= TOL["bf16"], ("prefill", err)
    saved = L.ring.save()
    start = w.prefix + w.T

    def sweep(seed, check):
        outs, e = [], 0.0
        Kd, Vd = Kh.copy(), Vh.copy()
        for s in range(w.decode_steps):
            tok = wl.decode_token(w, layer, s, seed=seed)
            p = start + s
            o_dev = L.decode(tok)
            outs.append(o_dev.view(torch.int16).clone())
            Kd[:, p - hb] = _rot(w, tok["k"], p)[:, 0]
            Vd[:, p - hb] = tok["v"][:, 0]
            if s in check:
                q_r = _rot(w, tok["q"], p)
                o = attend_query(q_r[0, 0], Kd[0], Vd[0], L.sinks_h, p - hb, W, w.sm_scale)
                e = max(e, max_abs(host(o_dev)[0, 0], o))
        torch.cuda.synchronize()
        return torch.stack(outs), e

    a1, e1 = sweep(0, set(range(w.decode_steps)))
    assert e1 <= TOL["bf16"], ("decode seed 0", e1)
    L.ring.load(saved)
    assert L.ring.offset == start
    b, e2 = sweep(1, {0, 31})
    assert e2 <= TOL["bf16"], ("decode seed 1", e2)
    L.ring.load(saved)
    a2, _ = sweep(0, set())
    assert torch.equal(a1, a2)
    assert not torch.equal(a1, b)
