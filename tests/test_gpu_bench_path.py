"""The handover workload exactly as bench.py times it -- its own layer state
and step (fused RoPE + append of the 2048-token chunk at offset 65,536,
sink attention of the chunk, snapshot, 32 decode steps, restore, 32 steps
under the other seed, both layers) -- against the fp64 oracle on sampled
outputs: chunk rows at the tile edges and the handover diagonal, and decode
steps of both sweeps (2e-2).  The oracle starts from the raw seeded draws
and its own RoPE."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle.attention import attend_query
from oracle.rounding import round_to
from oracle.yarn import rope_apply
from tests.gpu_helpers import TOL, host, max_abs, oracle_tables

pytestmark = pytest.mark.gpu
sa = pytest.importorskip("long_context_sparse_yarn_amd")


def _rot(w, x, offset):
    inv, c = oracle_tables(w.d_h, w.yarn)
    return round_to(rope_apply(np.asarray(x, np.float64), offset, inv, c), "bf16")


@pytest.mark.timeout(600)
def test_bench_handover_step_matches_oracle():
    import bench
    w = wl.HANDOVER
    layers = [bench.HandoverLayer(w, i, sa, torch) for i in range(len(w.windows))]
    bench.handover_step(layers, w, sa)
    torch.cuda.synchronize()
    base = w.prefix + w.T
    for L in layers:
        x = L.host
        q_rot = _rot(w, x["q"], w.prefix)
        k_rot = _rot(w, x["k"], w.prefix)
        K = np.concatenate([x["prefix_k"].astype(np.float64), k_rot], 1)
        V = np.concatenate([x["prefix_v"].astype(np.float64), x["v"].astype(np.float64)], 1)
        out = host(L.out)
        err = 0.0
        for t in (0, 1, 15, 16, 63, 64, 1023, w.T - 1):
            o = attend_query(q_rot[0, t], K[0], V[0], x["sinks"], w.prefix + t, L.window, w.sm_scale)
            err = max(err, max_abs(out[0, t], o))
        assert err <= TOL["bf16"], ("chunk", L.window, err)
        dout = host(L.dout)                       # [2, steps, B, 1, n_q, d]
        Kd = np.empty((1, base + w.decode_steps) + K.shape[2:])
        Vd = np.empty_like(Kd)
        Kd[:, :base], Vd[:, :base] = K, V
        for sweep in range(2):                            # restore: rows >= base are rewritten
            err = 0.0
            for s in range(w.decode_steps):
                tok = wl.decode_token(w, L.layer, s, seed=w.seed + sweep)
                p = base + s
                Kd[:, p] = _rot(w, tok["k"], p)[:, 0]
                Vd[:, p] = tok["v"][:, 0]
                if s in (0, 1, w.decode_steps - 1):       # step 0: the first query after the chunk
                    q_r = _rot(w, tok["q"], p)
                    o = attend_query(q_r[0, 0], Kd[0], Vd[0], x["sinks"], p, L.window, w.sm_scale)
                    err = max(err, max_abs(dout[sweep, s, 0, 0], o))
            assert err <= TOL["bf16"], ("decode", L.window, sweep, err)
    # the cache offset after the step: the chunk plus one sweep of tokens
    assert all(L.cache.offset == base + w.decode_steps for L in layers)
