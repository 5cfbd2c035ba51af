"""Throughput of the sink-GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-extra] [--no-cpu]

One step = the whole hot path over one batch of the prefill-to-decode
handover workload (the largest that fits one GPU): B=1, n_q=64, n_kv=8,
d_h=64, bf16, YaRN s=32 base 1.5e5, a cache pre-filled with 65,536 rows.
For each of its two layer kinds (128-token band, full causal): the cache
rewound to the prefix, RoPE of the 2048-token chunk's Q and K at positions
65,536.. with K/V appended in the same pass, sink attention of the chunk at
offset 65,536, and a snapshot; then 32 decode steps per layer (one fused
call per token: RoPE of its Q and K, append of its K/V row, sink attention
against the cache), a restore, and 32 more steps under another seed.  Inputs are resident in HBM before timing starts.
The value is algorithmic attention TFLOP/s of the step (4*d*n_q*B*sum_p|A(p)|
flops over the allowed query/key pairs of the chunk and of every decode
query).

Extra objects on the same JSON line:
  roofline      the full-causal prefill kernel of the chunk (the step's
                dominant kernel), timed with HIP events on its stream inside
                the timed steps, against dense bf16 MFMA
  decode_kv     the long-context decode workload's full-causal layer (B8,
                131,072 cached rows): KV GB/s of its attention kernels
  handover      per-layer prefill figures and the decode sweeps' figures
  cpu_baseline  the fp64 oracle on bounded samples: the handover step (the
                value) and, with the extras, the other prefill and decode
                workloads
  extra         GPT-OSS-Lite prefill (B4 T4096 8/4 d96) and gpt-oss prefill
                (B1 T8192 64/8 d64) steps, long-context decode per layer, and
                the fused projection, MoE layer and sampling figures
"""
import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)

# HBM bytes per launch of the roofline kernel, from rocprofv3 FETCH_SIZE x 2.0 +
# WRITE_SIZE x 1.0 (factors from a 512 MiB copy: FETCH_SIZE reads 256 MiB,
# WRITE_SIZE 512 MiB), keyed by (workload, window); valid only while the
# kernel sources hash to the value they were measured with.
TRAFFIC = {("handover", 0): {"sources_sha256_16": "5d319fe836e3b076", "bytes": 536790269}}
KERNEL_SOURCES = ("prefill.hip", "sa_device.h", "sa_attn.h", "sa_rope.h")   # what the prefill kernel is built from
KERNEL_REPEAT = 20             # back-to-back launches per kernel-duration measurement


def prefill_kernel_name(d, band):
    """Template instance sinkattn_prefill launches for head dim d (tile shape
    from the SA_PF* / SA_PFB* defaults in prefill.hip; `false`: Q arrives
    rotated; the last flag: a full-causal (long-walk) instance)."""
    src = open(os.path.join(ROOT, "long_context_sparse_yarn_amd", "csrc", "prefill.hip")).read()
    m = re.search(r"#define SA_PF%s%d (\d+), (\d+)" % ("B" if band else "", d), src)
    return ("prefill_bf16_kernel<%d,%s,%s,false,%s>" % (d, m.group(1), m.group(2),
                                                       "false" if band else "true") if m
            else "prefill_bf16_kernel<%d>" % d)


def kernel_sources_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_sparse_yarn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pairs_allowed(q_offset, T, window):
    p = q_offset + np.arange(T, dtype=np.int64)
    n = p + 1
    if window > 0:
        n = np.minimum(n, window)
    return int(n.sum())


def attn_flops(B, n_q, d, q_offset, T, window):
    return 4.0 * d * n_q * B * pairs_allowed(q_offset, T, window)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--extra-only", choices=("sampling", "moe", "qkv"), default=None,
                    help="print only that extra leg's figures (for profiling it alone)")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="oracle seconds per sampled workload")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="GPU clock settle before the warmup steps: back-to-back launches of "
                         "the step's full-causal prefill for this long (untimed)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized buffer 3 times (reference dispatch for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


class Layer:
    """Device state of one layer of a prefill workload."""

    def __init__(self, w, layer, sa, torch):
        import workloads as wl
        x = wl.prefill_inputs(w, layer)
        dt = torch.bfloat16
        up = lambda a: torch.from_numpy(a).cuda().to(dt)
        self.host = x
        self.window = w.windows[layer]
        self.q0, self.k0, self.v = up(x["q"]), up(x["k"]), up(x["v"])
        self.qw = torch.empty_like(self.q0)
        self.sinks = torch.from_numpy(x["sinks"]).cuda()
        self.cache = sa.KVCache.empty(w.B, w.capacity, w.n_kv, w.d_h, dtype=dt)
        if w.prefix:
            self.cache.append(up(x["prefix_k"]), up(x["prefix_v"]))
        self.snap = self.cache.snapshot()
        self.out = torch.empty_like(self.q0)
        self.yarn = sa.Yarn(w.d_h, w.yarn.base, w.yarn.factor, w.yarn.orig_ctx, w.yarn.alpha,
                            w.yarn.beta)


def run_layer(L, w, sa, ev=None):
    L.cache.restore(L.snap)
    o = L.cache.offset
    L.q_offset = o
    # Q rotated into qw and K into the cache at positions o.., V appended: one pass
    L.cache.append_rope_qk(L.q0, L.k0, L.v, L.yarn, q_out=L.qw)
    if ev is not None:
        ev[0].record()
    sa.sinkattn_prefill(L.qw, L.cache, L.sinks, L.window, w.sm_scale, o, out=L.out)
    if ev is not None:
        ev[1].record()


STEP_STATS = {}       # median and min per step (ms) from a pass after the timed steps
IN_STEP_STATS = {}    # timed layer: median and min of its in-step prefill launch (ms)


def time_prefill_step(w, sa, torch, steps, warmup):
    """Times `steps` steps after `warmup`.  Inside the timed region the only
    events are the two marks at its ends and one pair around the full-causal
    layer's prefill (the roofline kernel, timed live on its stream); each
    event record costs the step time (five per step measured 6% slower).
    Then each layer's prefill over KERNEL_REPEAT back-to-back launches, and
    a second pass of `steps` steps with an event at every step boundary for
    the per-step spread."""
    layers = [Layer(w, i, sa, torch) for i in range(len(w.windows))]
    full_i = [i for i, L in enumerate(layers) if L.window == 0][0]
    for _ in range(warmup):
        for L in layers:
            run_layer(L, w, sa)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        for i, L in enumerate(layers):
            run_layer(L, w, sa, evs[s] if i == full_i else None)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    live = [a.elapsed_time(b) for a, b in evs]
    in_step = {i: (float(np.mean(live)) if i == full_i else None) for i in range(len(layers))}
    IN_STEP_STATS.clear()
    IN_STEP_STATS[full_i] = (float(np.median(live)), float(np.min(live)))
    # Kernel durations: an event pair around one launch also spans its
    # dispatch and completion (several microseconds), so each layer's prefill
    # is also timed over KERNEL_REPEAT back-to-back launches on the step's
    # live buffers right after the timed steps (what a kernel trace reports).
    b2b = {}
    for i, L in enumerate(layers):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, KERNEL_REPEAT)   # a band layer's launch: about a call's host time
        a.record()
        for _ in range(KERNEL_REPEAT):
            sa.sinkattn_prefill(L.qw, L.cache, L.sinks, L.window, w.sm_scale, L.q_offset,
                                out=L.out)
        b.record()
        torch.cuda.synchronize()
        b2b[i] = a.elapsed_time(b) / KERNEL_REPEAT
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for s in range(steps):
        for L in layers:
            run_layer(L, w, sa)
        marks[s + 1].record()
    torch.cuda.synchronize()
    per_step = [marks[s].elapsed_time(marks[s + 1]) for s in range(steps)]
    STEP_STATS.clear()
    STEP_STATS.update(median=float(np.median(per_step)), min=float(np.min(per_step)))
    return layers, ms_step, b2b, in_step


class HandoverLayer:
    """Device state of one layer of the handover workload: the cache with its
    pre-filled prefix, the chunk's raw Q/K/V, and the decode tokens of both
    sweeps (seed 0, then seed 1)."""

    def __init__(self, w, layer, sa, torch):
        import workloads as wl
        x = wl.prefill_inputs(w, layer)
        dt = torch.bfloat16
        up = lambda a: torch.from_numpy(a).cuda().to(dt)
        self.host = x
        self.layer = layer
        self.window = w.windows[layer]
        self.q0, self.k0, self.v = up(x["q"]), up(x["k"]), up(x["v"])
        self.qw = torch.empty_like(self.q0)
        self.out = torch.empty_like(self.q0)
        self.sinks = torch.from_numpy(x["sinks"]).cuda()
        self.cache = sa.KVCache.empty(w.B, w.capacity, w.n_kv, w.d_h, dtype=dt)
        self.cache.append(up(x["prefix_k"]), up(x["prefix_v"]))
        self.snap0 = self.cache.snapshot()
        self.snap1 = None
        self.yarn = sa.Yarn(w.d_h, w.yarn.base, w.yarn.factor, w.yarn.orig_ctx, w.yarn.alpha,
                            w.yarn.beta)
        self.toks = [[{k: up(a) for k, a in wl.decode_token(w, layer, s, seed=w.seed + sw).items()}
                      for s in range(w.decode_steps)] for sw in range(2)]
        self.qtok = torch.empty_like(self.toks[0][0]["q"])
        self.dout = torch.empty((2, w.decode_steps) + tuple(self.qtok.shape), dtype=dt,
                                device="cuda")
        self.ws = sa.decode_workspace(self.cache, w.n_q)

    def prefill(self, w, sa, ev=None):
        self.cache.restore(self.snap0)
        self.cache.append_rope_qk(self.q0, self.k0, self.v, self.yarn, q_out=self.qw)
        if ev is not None:
            ev[0].record()
        sa.sinkattn_prefill(self.qw, self.cache, self.sinks, self.window, w.sm_scale, w.prefix,
                            out=self.out)
        if ev is not None:
            ev[1].record()
        self.snap1 = self.cache.snapshot()

    def decode(self, w, sa, sweep, s):
        """The fused step: RoPE of the token's Q and K, append of its K/V row
        and sink attention in one call (bit-equal to append_rope_qk +
        sinkattn_decode)."""
        t = self.toks[sweep][s]
        sa.sinkattn_decode_step(self.cache, t["q"], t["k"], t["v"], self.sinks, self.window,
                                w.sm_scale, self.yarn, workspace=self.ws, out=self.dout[sweep, s])


def handover_step(layers, w, sa, ev=None, sweep_ev=None):
    """One step of the handover workload: both layers' chunk prefill (each
    ending with a snapshot), then two decode sweeps, each starting from a
    restore of that snapshot; within a sweep, token s runs through both
    layers before token s+1."""
    for L in layers:
        L.prefill(w, sa, ev if (ev is not None and L.window == 0) else None)
    for sweep in range(2):
        if sweep_ev is not None:
            sweep_ev[sweep][0].record()
        for L in layers:
            L.cache.restore(L.snap1)
        for s in range(w.decode_steps):
            for L in layers:
                L.decode(w, sa, sweep, s)
        if sweep_ev is not None:
            sweep_ev[sweep][1].record()


def handover_flops(w):
    """(prefill flops per layer kind, decode flops per layer kind) of one step."""
    pre = {W: attn_flops(w.B, w.n_q, w.d_h, w.prefix, w.T, W) for W in w.windows}
    base = w.prefix + w.T
    dec = {W: 2 * sum(attn_flops(w.B, w.n_q, w.d_h, base + s, 1, W) for s in range(w.decode_steps))
           for W in w.windows}
    return pre, dec


def decode_bytes(w, pos, W):
    """Algorithmic bytes of one decode attention call at query position pos:
    each allowed K and V row once, q read, out written (bf16)."""
    rows = min(pos + 1, W) if W > 0 else pos + 1
    return (rows * w.n_kv * w.d_h * 2 * 2 + 2 * w.n_q * w.d_h * 2) * w.B


def settle_clock(fn, torch, ms):
    """Back-to-back launches of fn for about `ms` milliseconds (untimed), so
    the timed steps start at the clock the GPU holds under this load."""
    if ms <= 0:
        return 0
    t_end = time.perf_counter() + ms * 1e-3
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
    return n


def time_handover(w, sa, torch, steps, warmup, settle_ms):
    """Times exactly `steps` handover steps after `warmup` untimed ones (and
    the clock settle).  The only events inside the timed region are its two
    end marks and one pair around the full-causal prefill launch of each
    step (the roofline kernel, live on its stream).  A second pass of the
    same steps, after the timed region, carries events at the step
    boundaries (spread) and around each decode sweep."""
    layers = [HandoverLayer(w, i, sa, torch) for i in range(len(w.windows))]
    full = [L for L in layers if L.window == 0][0]
    full.prefill(w, sa)
    n_settle = settle_clock(lambda: sa.sinkattn_prefill(full.qw, full.cache, full.sinks, 0,
                                                        w.sm_scale, w.prefix, out=full.out),
                            torch, settle_ms)
    for _ in range(warmup):
        handover_step(layers, w, sa)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(E(), E()) for _ in range(steps)]
    t0, t1 = E(), E()
    torch.cuda.synchronize()
    t0.record()
    for k in range(steps):
        handover_step(layers, w, sa, ev=evs[k])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    live = [a.elapsed_time(b) for a, b in evs]
    # second pass: step spread and decode sweeps
    marks = [E() for _ in range(steps + 1)]
    sweeps = [[(E(), E()), (E(), E())] for _ in range(steps)]
    marks[0].record()
    for k in range(steps):
        handover_step(layers, w, sa, sweep_ev=sweeps[k])
        marks[k + 1].record()
    torch.cuda.synchronize()
    per_step = [marks[k].elapsed_time(marks[k + 1]) for k in range(steps)]
    sweep_ms = [a.elapsed_time(b) for sw in sweeps for a, b in sw]
    # each layer's prefill over back-to-back launches on the live buffers
    b2b = {}
    for L in layers:
        L.prefill(w, sa)
        a, b = E(), E()
        queue_ahead(torch, KERNEL_REPEAT)   # a band layer's launch: about a call's host time
        a.record()
        for _ in range(KERNEL_REPEAT):
            sa.sinkattn_prefill(L.qw, L.cache, L.sinks, L.window, w.sm_scale, w.prefix, out=L.out)
        b.record()
        torch.cuda.synchronize()
        b2b[L.window] = a.elapsed_time(b) / KERNEL_REPEAT
    # leave every layer as a step leaves it (outputs of the last step)
    handover_step(layers, w, sa)
    torch.cuda.synchronize()
    return {"layers": layers, "ms_step": ms_step, "live": live, "per_step": per_step,
            "sweep_ms": sweep_ms, "b2b": b2b, "settle_launches": n_settle}


def handover_figures(w, t):
    pre, dec = handover_flops(w)
    layers = []
    for L in t["layers"]:
        ms = float(np.mean(t["live"])) if L.window == 0 else t["b2b"][L.window]
        f = prefill_figures(w, L, t["b2b"][L.window], ms if L.window == 0 else None)
        if L.window == 0:
            f["kernel_ms_in_step_median"] = round(float(np.median(t["live"])), 4)
            f["kernel_ms_in_step_min"] = round(float(np.min(t["live"])), 4)
        layers.append(f)
    base = w.prefix + w.T
    by_sweep = sum(decode_bytes(w, base + s, W) for s in range(w.decode_steps) for W in w.windows)
    fl_sweep = sum(dec.values()) / 2
    sw = float(np.mean(t["sweep_ms"]))
    return {"layers": layers,
            "decode_sweep": {"steps": w.decode_steps, "layers": len(w.windows),
                             "ms": round(sw, 4), "us_per_token": round(sw * 1e3 / w.decode_steps, 2),
                             "alg_mb": round(by_sweep / 1e6, 2),
                             "gbs": round(by_sweep / (sw * 1e-3) / 1e9, 1),
                             "frac_hbm": round(by_sweep / (sw * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "gflop": round(fl_sweep / 1e9, 3),
                             "timing": "events around each sweep (restore, then per token and layer "
                                       "fused RoPE + append + sink attention), second pass",
                             "cache_note": "each step re-reads the same ~138 MB of K/V, which fits "
                                           "the 256 MB Infinity Cache: frac_hbm is against the HBM "
                                           "peak, but reads may be served from that cache"},
            "gflop_step": {"prefill": {str(k): round(v / 1e9, 2) for k, v in pre.items()},
                           "decode": {str(k): round(v / 1e9, 3) for k, v in dec.items()}}}


def abi_call_figures(w, L, sa, torch):
    """Each data-moving ABI call of a prefill layer timed on its own (events
    around KERNEL_REPEAT back-to-back calls on the layer's buffers), in
    algorithmic GB/s: RoPE of Q out of place, the plain append, and the fused
    rotate-Q-and-K-and-append pass the step uses."""
    elt = 2
    qb = w.B * w.T * w.n_q * w.d_h * elt
    kvb = 2 * w.B * w.T * w.n_kv * w.d_h * elt
    kr = torch.empty_like(L.k0)
    sa.yarn_rope_apply(L.k0, L.q_offset, L.yarn, out=kr)
    calls = {
        "yarn_rope(q)": (lambda: sa.yarn_rope_apply(L.q0, L.q_offset, L.yarn, out=L.qw), 2 * qb),
        "kv_cache_append": (lambda: (L.cache.restore(L.snap), L.cache.append(kr, L.v)), 2 * kvb),
        "kv_cache_append_rope_qk": (lambda: (L.cache.restore(L.snap),
                                             L.cache.append_rope_qk(L.q0, L.k0, L.v, L.yarn,
                                                                    q_out=L.qw)),
                                    2 * qb + 2 * kvb),
    }
    out = {}
    for name, (fn, by) in calls.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, 2 * KERNEL_REPEAT)   # (a restore and a call each)
        a.record()
        for _ in range(KERNEL_REPEAT):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / KERNEL_REPEAT * 1e3
        out[name] = {"us": round(us, 2), "alg_mb": round(by / 1e6, 2),
                     "gbs": round(by / (us * 1e-6) / 1e9, 1),
                     "frac_hbm": round(by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    # leave the layer as the step left it (rotated Q, appended cache)
    run_layer(L, w, sa)
    torch.cuda.synchronize()
    return out


def ring_prefill_figures(w, L, sa, torch):
    """The band layer through a W-row ring instead of a T-row cache: stage
    (nothing to copy at offset 0), fused RoPE + append into the stage,
    prefill over the stage, commit of the last W rows into the ring; timed
    over KERNEL_REPEAT back-to-back layer passes against the same passes on
    the linear cache.  KV bytes are the caches' logical bf16 entries."""
    W, dt = L.window, torch.bfloat16
    kbuf = torch.empty((w.B, W, w.n_kv, w.d_h), dtype=dt, device="cuda")
    vbuf = torch.empty(sa.v_cache_shape(w.B, W, w.n_kv, w.d_h), dtype=dt, device="cuda")
    stage_rows = ((W - 1 + w.T + 31) // 32) * 32
    stage = sa.KVCache.empty(w.B, stage_rows, w.n_kv, w.d_h, dtype=dt)
    out = torch.empty_like(L.out)

    def ring_pass():
        ring = sa.KVRing(kbuf, vbuf)          # an empty ring over the same buffers (host only)
        ring.stage(stage)
        stage.append_rope_qk(L.q0, L.k0, L.v, L.yarn, q_out=L.qw)
        sa.sinkattn_prefill(L.qw, stage, L.sinks, W, w.sm_scale, 0, out=out)
        ring.commit(stage)
        return ring

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, 5 * KERNEL_REPEAT)   # (up to five calls a pass)
        a.record()
        for _ in range(KERNEL_REPEAT):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / KERNEL_REPEAT

    ring_ms = timed(ring_pass)
    lin_ms = timed(lambda: run_layer(L, w, sa))
    same = bool(torch.equal(out.view(torch.int16), L.out.view(torch.int16)))
    row = w.n_kv * w.d_h * 2 * 2                     # K + V bytes of one position
    n_layers = 12
    full_b = w.B * w.capacity * row
    return {"window": W, "layer_ms_ring": round(ring_ms, 4), "layer_ms_linear": round(lin_ms, 4),
            "out_bitequal_linear": same,
            "kv_bytes": {"band_layer_linear": w.B * w.capacity * row,
                         "band_layer_ring": w.B * W * row,
                         "stage_scratch_shared": w.B * stage_rows * row,
                         "full_layer": full_b,
                         "reduction_%d_alternating_layers" % n_layers:
                             round((n_layers * full_b) /
                                   (n_layers // 2 * full_b + n_layers // 2 * w.B * W * row), 4)}}


def prefill_figures(w, L, ms_b2b, ms_in_step=None):
    """Figures of one layer's prefill kernel from its live in-step duration
    where the timed steps measured it, else from back-to-back launches."""
    ms = ms_in_step if ms_in_step is not None else ms_b2b
    fl = attn_flops(w.B, w.n_q, w.d_h, w.prefix, w.T, L.window)
    elt = 2
    # algorithmic bytes: Q read + O written + each allowed K/V row read once
    lo = max(0, w.prefix - L.window + 1) if L.window > 0 else 0
    rows = (w.prefix + w.T) - lo
    by = (2 * w.B * w.T * w.n_q * w.d_h + 2 * w.B * rows * w.n_kv * w.d_h) * elt
    tf = fl / (ms * 1e-3) / 1e12
    gbs = by / (ms * 1e-3) / 1e9
    return {"window": L.window, "kernel_ms": round(ms, 4),
            "kernel_timing": "live in the timed steps" if ms_in_step is not None else "back to back",
            "kernel_ms_back_to_back": round(ms_b2b, 4),
            "gflop": round(fl / 1e9, 3),
            "tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4),
            "alg_mb": round(by / 1e6, 2), "gbs": round(gbs, 1),
            "frac_bound": round(tf / min(PEAK_BF16_TFLOPS, fl / by * PEAK_HBM_GBS / 1e3), 4)}


def queue_ahead(torch, calls):
    """Queue a spin kernel (torch's) about as long as the host needs to issue
    `calls` library calls (30 us each at most, at 2.4 GHz), so that the
    launches issued next wait behind it: the events between them then time
    the GPU's work, not the Python loop that issues the calls (a band-layer
    decode kernel runs in a few microseconds, and a band-layer prefill or a
    RoPE pass in ten to twenty, about what a call costs the host).  No longer
    than that: a GPU left nearly idle behind a long spin lowers its clock."""
    torch.cuda._sleep(int(calls * 30e-6 * 2.4e9))


def decode_back_to_back(sa, torch, q, cache, sinks, W, sm_scale, ws, out):
    """ms per sinkattn_decode launch, KERNEL_REPEAT launches between one pair
    of events (queued behind a spin kernel): the cache as the last step left
    it and that step's rotated Q, so every launch does that step's work."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    queue_ahead(torch, KERNEL_REPEAT)
    a.record()
    for _ in range(KERNEL_REPEAT):
        sa.sinkattn_decode(q, cache, sinks, W, sm_scale, workspace=ws, out=out)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / KERNEL_REPEAT


def ring_decode_figures(w, W, pk, pv, sinks, toks, y, sa, torch):
    """The band layer's decode steps on a W-row ring holding the prefix's last
    W rows (appending the whole prefix keeps only those), restored by
    kv_ring_load between the warmup and the timed steps."""
    ring = sa.KVRing.empty(w.B, W, w.n_kv, w.d_h, dtype=torch.bfloat16)
    ring.append(pk, pv)
    saved = ring.save()
    ws = sa.decode_workspace(ring, w.n_q)
    qbuf = torch.empty_like(toks[0]["q"])
    out = torch.empty_like(qbuf)

    def step(s, ev=None):
        ring.append_rope_qk(toks[s]["q"], toks[s]["k"], toks[s]["v"], y, q_out=qbuf)
        if ev is not None:
            ev[0].record()
        sa.sinkattn_decode(qbuf, ring, sinks, W, w.sm_scale, workspace=ws, out=out)
        if ev is not None:
            ev[1].record()

    for s in range(4):
        step(s)
    ring.load(saved)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.decode_steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead(torch, 2 * w.decode_steps)
    t0.record()
    for s in range(w.decode_steps):
        step(s, evs[s])
    t1.record()
    torch.cuda.synchronize()
    kms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    step_ms = t0.elapsed_time(t1) / w.decode_steps
    b2b_ms = decode_back_to_back(sa, torch, qbuf, ring, sinks, W, w.sm_scale, ws, out)
    return {"attn_kernel_us": round(kms * 1e3, 2),
            "attn_kernel_us_back_to_back": round(b2b_ms * 1e3, 2),
            "step_us": round(step_ms * 1e3, 2),
            "kv_bytes": w.B * W * w.n_kv * w.d_h * 2 * 2}


def decode_extra(sa, torch, steps_warm=4):
    import workloads as wl
    w = wl.LONG_DECODE
    dt = torch.bfloat16
    up = lambda a: torch.from_numpy(a).cuda().to(dt)
    res = {}
    pre = wl.prefix_inputs(w, 0)
    pk, pv = up(pre["prefix_k"]), up(pre["prefix_v"])
    del pre
    y = sa.Yarn(w.d_h, w.yarn.base, w.yarn.factor, w.yarn.orig_ctx, w.yarn.alpha, w.yarn.beta)
    for layer, W in enumerate(w.windows):
        cache = sa.KVCache.empty(w.B, w.capacity, w.n_kv, w.d_h, dtype=dt)
        cache.append(pk, pv)             # the band layer reuses the full layer's prefix draw
        sinks = torch.from_numpy(wl.sinks(w, layer)).cuda()
        toks = [wl.decode_token(w, layer, s) for s in range(w.decode_steps)]
        toks = [{k: up(v) for k, v in t.items()} for t in toks]
        ws = sa.decode_workspace(cache, w.n_q)
        snap = cache.snapshot()
        qbuf = torch.empty_like(toks[0]["q"])
        out = torch.empty_like(qbuf)

        def step(s, ev=None):
            cache.append_rope_qk(toks[s]["q"], toks[s]["k"], toks[s]["v"], y, q_out=qbuf)
            if ev is not None:
                ev[0].record()
            sa.sinkattn_decode(qbuf, cache, sinks, W, w.sm_scale, workspace=ws, out=out)
            if ev is not None:
                ev[1].record()

        for s in range(steps_warm):
            step(s)
        cache.restore(snap)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(w.decode_steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, 2 * w.decode_steps)
        t0.record()
        for s in range(w.decode_steps):
            step(s, evs[s])
        t1.record()
        torch.cuda.synchronize()
        kms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        step_ms = t0.elapsed_time(t1) / w.decode_steps
        # the same steps through the fused entry point (one call per token)
        cache.restore(snap)
        for s in range(steps_warm):
            sa.sinkattn_decode_step(cache, toks[s]["q"], toks[s]["k"], toks[s]["v"], sinks, W,
                                    w.sm_scale, y, workspace=ws, out=out)
        cache.restore(snap)
        torch.cuda.synchronize()
        queue_ahead(torch, w.decode_steps)
        t0.record()
        for s in range(w.decode_steps):
            sa.sinkattn_decode_step(cache, toks[s]["q"], toks[s]["k"], toks[s]["v"], sinks, W,
                                    w.sm_scale, y, workspace=ws, out=out)
        t1.record()
        torch.cuda.synchronize()
        fused_ms = t0.elapsed_time(t1) / w.decode_steps
        b2b_ms = decode_back_to_back(sa, torch, qbuf, cache, sinks, W, w.sm_scale, ws, out)
        rows = [min(w.prefix + s + 1, W) if W > 0 else w.prefix + s + 1
                for s in range(w.decode_steps)]
        by = np.mean([(r * w.n_kv * w.d_h * 2 * 2 + 2 * w.n_q * w.d_h * 2) * w.B for r in rows])
        gbs = by / (kms * 1e-3) / 1e9
        res["full" if W == 0 else "band%d" % W] = {
            "attn_kernel_us": round(kms * 1e3, 2),
            "attn_kernel_us_back_to_back": round(b2b_ms * 1e3, 2),
            "step_us": round(step_ms * 1e3, 2),
            "fused_step_us": round(fused_ms * 1e3, 2),
            "alg_mb_per_step": round(by / 1e6, 3), "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "kv_bytes": w.B * w.capacity * w.n_kv * w.d_h * 2 * 2}
        if W > 0:
            res["band%d_ring" % W] = ring_decode_figures(w, W, pk, pv, sinks, toks, y, sa, torch)
        del cache, ws, toks
        torch.cuda.empty_cache()
    return {"workload": w.name, **res,
            "timing": "attn_kernel_us: events around each step's attention launches (the "
                      "events' own cost included: ~2-3 us, which dominates a band layer's figure); "
                      "attn_kernel_us_back_to_back: %d attention launches at the last step's state "
                      "between one pair of events; step_us: " % KERNEL_REPEAT +
                      "the separate calls (append_rope_qk, then decode) per step; fused_step_us: "
                      "sinkattn_decode_step per step; each over 64 steps queued behind a spin "
                      "kernel, so the events time the GPU, not the host's calls"}


QKV_D_MODEL = {"gpt-oss": 2880, "gpt-oss-lite": 768}   # residual widths (study note; visual guide)


def qkv_extra(sa, torch):
    """The fused qkv projection with the RoPE + append epilogue
    (sinkattn_qkv_rope_append) on the two prefill workloads' shapes, seeded
    random bf16 weights: TFLOP/s of the projection (2 B T d_qkv d_model per
    launch), against the same step done as torch's bf16 linear (the
    library GEMM) followed by kv_cache_append_rope_qk."""
    import workloads as wl
    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    for w, key in ((wl.GPTOSS_PREFILL, "gpt-oss"), (wl.LITE_PREFILL, "gpt-oss-lite")):
        dm = QKV_D_MODEL[key]
        y = sa.Yarn(w.d_h, w.yarn.base, w.yarn.factor, w.yarn.orig_ctx, w.yarn.alpha, w.yarn.beta)
        N = w.d_h * (w.n_q + 2 * w.n_kv)
        x = torch.randn(w.B, w.T, dm, device="cuda", generator=g).to(torch.bfloat16)
        W = (torch.randn(N, dm, device="cuda", generator=g) / dm ** 0.5).to(torch.bfloat16)
        b = (0.1 * torch.randn(N, device="cuda", generator=g)).to(torch.bfloat16)
        c = sa.KVCache.empty(w.B, w.capacity, w.n_kv, w.d_h)
        snap = c.snapshot()
        qo = torch.empty(w.B, w.T, w.n_q, w.d_h, device="cuda", dtype=torch.bfloat16)
        ws = torch.empty(sa.qkv_workspace_bytes(w.T, w.d_h), dtype=torch.uint8, device="cuda")

        def fused():
            c.restore(snap)
            sa.qkv_rope_append(c, x, W, b, w.n_q, y, q_out=qo, workspace=ws)

        def separate():
            c.restore(snap)
            qkv = torch.nn.functional.linear(x, W, b)
            q = qkv[..., :w.n_q * w.d_h].reshape(w.B, w.T, w.n_q, w.d_h).contiguous()
            k = qkv[..., w.n_q * w.d_h:(w.n_q + w.n_kv) * w.d_h].reshape(
                w.B, w.T, w.n_kv, w.d_h).contiguous()
            v = qkv[..., (w.n_q + w.n_kv) * w.d_h:].reshape(w.B, w.T, w.n_kv, w.d_h).contiguous()
            c.append_rope_qk(q, k, v, y, q_out=qo)

        fl = 2.0 * w.B * w.T * N * dm
        res = {"B": w.B, "T": w.T, "d_model": dm, "d_qkv": N, "gflop": round(fl / 1e9, 2)}
        for nm, f in (("fused", fused), ("torch_linear_then_append_rope_qk", separate)):
            f()
            torch.cuda.synchronize()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            for _ in range(KERNEL_REPEAT):
                f()
            b_.record()
            torch.cuda.synchronize()
            us = a_.elapsed_time(b_) / KERNEL_REPEAT * 1e3
            res[nm] = {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1),
                       "frac_mfma": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        out[key] = res
        del x, W, b, c, qo, ws
        torch.cuda.empty_cache()
    return out


# GPT-OSS-Lite MoE layer (visual guide, Architecture Specifications): 8 routed
# SwiGLU experts of width 1536, top 2, one shared expert, d_model 768, on the
# prefill workload's 4 x 4096 tokens
MOE_LITE = {"N": 4 * 4096, "d_model": 768, "E": 8, "k": 2, "ffn": 1536, "ffn_shared": 1536}


def moe_extra(sa, torch):
    """moe_layer on the GPT-OSS-Lite MoE shape with seeded random bf16
    weights: TFLOP/s of the expert GEMMs actually run (router, N k routed
    rows through gate, up and down, N rows through the shared expert),
    against the same layer written with torch ops (bf16 linears, topk,
    one masked gather per expert)."""
    c = MOE_LITE
    N, dm, E, k, ffn, fs = c["N"], c["d_model"], c["E"], c["k"], c["ffn"], c["ffn_shared"]
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    rn = lambda *sh, fan: (torch.randn(*sh, device="cuda", generator=g) / fan ** 0.5).to(torch.bfloat16)
    x = torch.randn(N, dm, device="cuda", generator=g).to(torch.bfloat16)
    wr, w13, w2 = rn(E, dm, fan=dm), rn(E, 2 * ffn, dm, fan=dm), rn(E, dm, ffn, fan=ffn)
    w13s, w2s = rn(2 * fs, dm, fan=dm), rn(dm, fs, fan=fs)
    ws = torch.empty(sa.moe_workspace_bytes(N, dm, E, k, ffn, fs), dtype=torch.uint8, device="cuda")
    y = torch.empty(N, dm, dtype=torch.bfloat16, device="cuda")

    def fused():
        sa.moe_layer(x, wr, w13, w2, k, shared=(w13s, w2s), out=y, workspace=ws)

    def torch_layer():
        logits = torch.nn.functional.linear(x, wr)
        val, idx = torch.topk(logits.float(), k, dim=1)
        wts = torch.softmax(val, dim=1)
        acc = torch.zeros(N, dm, dtype=torch.float32, device="cuda")
        for e in range(E):
            tok, slot = (idx == e).nonzero(as_tuple=True)
            xe = x[tok]
            gu = torch.nn.functional.linear(xe, w13[e])
            h = (torch.nn.functional.silu(gu[:, :ffn].float()) * gu[:, ffn:].float()).to(torch.bfloat16)
            acc.index_add_(0, tok, wts[tok, slot][:, None] * torch.nn.functional.linear(h, w2[e]).float())
        gu = torch.nn.functional.linear(x, w13s)
        h = (torch.nn.functional.silu(gu[:, :fs].float()) * gu[:, fs:].float()).to(torch.bfloat16)
        return (acc + torch.nn.functional.linear(h, w2s).float()).to(torch.bfloat16)

    fl = 2.0 * N * dm * E + 2.0 * N * k * (2 * ffn * dm + ffn * dm) + 2.0 * N * (2 * fs * dm + fs * dm)
    res = {"workload": "GPT-OSS-Lite MoE: %d tokens, d_model %d, %d experts top %d, SwiGLU %d, "
                       "shared %d" % (N, dm, E, k, ffn, fs), "gflop": round(fl / 1e9, 2)}
    for nm, f in (("moe_layer", fused), ("torch_ops", torch_layer)):
        f()
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = KERNEL_REPEAT if nm == "moe_layer" else 5
        a_.record()
        for _ in range(reps):
            f()
        b_.record()
        torch.cuda.synchronize()
        us = a_.elapsed_time(b_) / reps * 1e3
        res[nm] = {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1),
                   "frac_mfma": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    del x, wr, w13, w2, w13s, w2s, ws, y
    torch.cuda.empty_cache()
    return res


SAMPLE_CONFIGS = [
    # name, params (per row), penalties from a 64-token history
    ("example request (T 0.2, top-p 0.95, min-p 0.05) + penalties",
     dict(temperature=0.2, top_p=0.95, min_p=0.05, repetition=1.1, presence=0.2, frequency=0.1)),
    ("top-k 50, T 0.7", dict(temperature=0.7, top_k=50)),
    ("top-p 0.9, T 1.0", dict(temperature=1.0, top_p=0.9)),
    ("no truncation, T 1.0", dict(temperature=1.0)),
    ("greedy", dict(temperature=0.0)),
]


def sample_extra(sa, torch):
    """sample_tokens on rows of fp32 logits over the GPT-OSS-Lite vocabulary
    (128,000) at the decode batch (8) and at 64 rows: microseconds per call
    (all three launches), tokens/s, and HBM GB/s of the inputs it must read
    (logits, plus the int32 counts when penalties are on), against the same
    controls written with torch ops (sort, cumsum, masks, inverse CDF)."""
    import workloads as wl
    res = {"vocab": wl.SAMPLE_V, "configs": []}
    for B in (wl.SAMPLE_B, 64):
        d = wl.sampling_inputs(B, wl.SAMPLE_V, seed=1)
        lg = torch.from_numpy(d["logits"]).cuda()
        ut = torch.from_numpy(d["u"]).cuda()
        counts = torch.zeros((B, wl.SAMPLE_V), dtype=torch.int32, device="cuda")
        sa.sample_count_tokens(torch.from_numpy(d["history"]).cuda(), counts)
        ws = torch.empty(sa.sample_workspace_bytes(B, wl.SAMPLE_V), dtype=torch.uint8, device="cuda")
        for name, p in SAMPLE_CONFIGS:
            if B != wl.SAMPLE_B and not name.startswith("example"):
                continue
            params = sa.sample_params(B, **p)
            pen = any(k in p for k in ("repetition", "presence", "frequency"))
            ct = counts if pen else None

            def run():
                sa.sample_tokens(lg, params, ut, counts=ct, workspace=ws)

            def torch_ops():
                z = lg
                if ct is not None:
                    seen = ct > 0
                    z = torch.where(seen, torch.where(z > 0, z / p["repetition"], z * p["repetition"]), z)
                    z = z - p["presence"] * seen.float() - p["frequency"] * ct.float()
                if p["temperature"] == 0.0:
                    return z.argmax(dim=1)
                pr = torch.softmax(z / p["temperature"], dim=1)
                ps, idx = torch.sort(pr, dim=1, descending=True)
                keep = torch.ones_like(ps, dtype=torch.bool)
                if p.get("top_k", 0):
                    keep[:, p["top_k"]:] = False
                if p.get("top_p", 1.0) < 1.0:
                    c = torch.cumsum(ps, dim=1)
                    keep &= (c - ps) < p["top_p"]
                if p.get("min_p", 0.0) > 0.0:
                    keep &= ps >= p["min_p"] * ps[:, :1]
                ps = ps * keep
                c = torch.cumsum(ps, dim=1)
                j = torch.searchsorted(c, (ut * c[:, -1]).unsqueeze(1)).clamp(max=ps.shape[1] - 1)
                return idx.gather(1, j)

            by = B * wl.SAMPLE_V * (8 if pen else 4)
            row = {"config": name, "B": B}
            for nm, f, reps in (("sample_tokens", run, KERNEL_REPEAT), ("torch_ops", torch_ops, 5)):
                f()
                torch.cuda.synchronize()
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
                for _ in range(reps):
                    f()
                b_.record()
                torch.cuda.synchronize()
                us = a_.elapsed_time(b_) / reps * 1e3
                row[nm] = {"us": round(us, 1), "tokens_per_s": round(B / us * 1e6, 0),
                           "gbs": round(by / us / 1e3, 1), "frac_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 4)}
            res["configs"].append(row)
        del lg, ut, counts, ws
    torch.cuda.empty_cache()
    return res


def _cpu_info():
    from threadpoolctl import threadpool_info
    info = threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] + [1])
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return int(cores), model


def cpu_prefill_sample(w, layers, budget_s, extra_flops=None):
    """The oracle as it stands on a bounded sample of a prefill step: RoPE
    of all of the chunk's Q and K (fp64), the append (the oracle's cache is
    the prefix with the rotated chunk after it), and attention of seeded
    random query rows (all heads) per layer.  Each layer's time is
    extrapolated from its own sampled rows by algorithmic flops (a band
    row and a full-causal row cost the oracle differently per flop);
    extra_flops {window: flops} adds a layer's decode queries of the step,
    which cost the oracle what its prefill rows of the same span do.  Also
    returns the largest difference between the sampled oracle rows and the
    GPU's output rows."""
    from oracle.attention import attend_query
    from oracle.rounding import round_to
    from oracle.yarn import rope_apply, yarn_concentration, yarn_inv_freq

    y = w.yarn
    inv = yarn_inv_freq(w.d_h, y.base, y.factor, y.orig_ctx, y.alpha, y.beta)
    c = yarn_concentration(y.factor)
    rng = np.random.default_rng(0)
    t_fixed = 0.0
    est = 0.0
    fl_total = fl_sampled = 0.0
    n_rows = 0
    t_rows = 0.0
    checks = []
    per_layer = budget_s / len(layers)
    for L in layers:
        x = L.host
        t = time.perf_counter()
        q_rot = round_to(rope_apply(x["q"].astype(np.float64), w.prefix, inv, c), "bf16")
        k_rot = round_to(rope_apply(x["k"].astype(np.float64), w.prefix, inv, c), "bf16")
        if w.prefix:
            K = np.concatenate([x["prefix_k"].astype(np.float64), k_rot], axis=1)
            V = np.concatenate([x["prefix_v"].astype(np.float64), x["v"].astype(np.float64)], axis=1)
        else:
            K, V = k_rot, x["v"]
        t_fixed += time.perf_counter() - t
        fl_layer = attn_flops(w.B, w.n_q, w.d_h, w.prefix, w.T, L.window)
        if extra_flops:
            fl_layer += extra_flops.get(L.window, 0.0)
        out_gpu = L.out.float().cpu().numpy()
        t_attn = fl_sample = 0.0
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < per_layer or fl_sample == 0.0:
            b = int(rng.integers(w.B))
            tq = int(rng.integers(w.T))
            p = w.prefix + tq
            t = time.perf_counter()
            o = attend_query(q_rot[b, tq], K[b], V[b], x["sinks"], p, L.window, w.sm_scale)
            t_attn += time.perf_counter() - t
            n = min(p + 1, L.window) if L.window > 0 else p + 1
            fl_sample += 4.0 * w.d_h * w.n_q * n
            n_rows += 1
            checks.append(float(np.max(np.abs(o - out_gpu[b, tq]))))
        est += t_attn * (fl_layer / fl_sample)
        fl_total += fl_layer
        fl_sampled += fl_sample
        t_rows += t_attn
        del K, V
    est += t_fixed
    return {"value": round(fl_total / est / 1e12, 6), "unit": "TFLOP/s", "est_step_s": round(est, 2),
            "sample": "fp64 numpy oracle on %s: RoPE of all Q and K of the chunk and the append "
                      "(%.2f s) plus attention of %d seeded random query rows (all heads, %.2f s, "
                      "%.3g of the step's flops); each layer's time extrapolated from its own rows "
                      "by flops" % (w.name, t_fixed, n_rows, t_rows, fl_sampled / fl_total),
            "parity_sample_max_abs": round(max(checks), 5) if checks else None}


def cpu_decode_sample(w, budget_s):
    """The oracle on the long-context decode workload: one decode query (all
    heads of one sequence) of the full layer at the first step's position,
    against sequence 0's pre-filled rows (drawn as the GPU run draws them)
    plus the appended row, timed repeatedly; the 64 steps of all sequences
    of both layers are extrapolated by algorithmic bytes (the oracle's cost
    is the pass over the allowed rows)."""
    import workloads as wl
    from oracle.attention import attend_query
    from oracle.rounding import round_to
    from oracle.yarn import rope_apply, yarn_concentration, yarn_inv_freq

    y = w.yarn
    inv = yarn_inv_freq(w.d_h, y.base, y.factor, y.orig_ctx, y.alpha, y.beta)
    c = yarn_concentration(y.factor)
    pk = wl.normal((1, w.prefix, w.n_kv, w.d_h), w.dtype, w.seed, w.cfg_idx, 0, wl.T_PREFIX_K)
    pv = wl.normal((1, w.prefix, w.n_kv, w.d_h), w.dtype, w.seed, w.cfg_idx, 0, wl.T_PREFIX_V)
    tok = wl.decode_token(w, 0, 0)
    t = time.perf_counter()
    p = w.prefix
    q_rot = round_to(rope_apply(tok["q"][:1].astype(np.float64), p, inv, c), "bf16")
    k_rot = round_to(rope_apply(tok["k"][:1].astype(np.float64), p, inv, c), "bf16")
    K = np.concatenate([pk.astype(np.float64), k_rot], axis=1)
    V = np.concatenate([pv.astype(np.float64), tok["v"][:1].astype(np.float64)], axis=1)
    t_fixed = time.perf_counter() - t
    sinks = wl.sinks(w, 0)
    n, t_attn = 0, 0.0
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < budget_s or n == 0:
        t = time.perf_counter()
        attend_query(q_rot[0, 0], K[0], V[0], sinks, p, 0, w.sm_scale)
        t_attn += time.perf_counter() - t
        n += 1
    by_call = decode_bytes(w.with_(B=1), p, 0)
    by_total = sum(decode_bytes(w, w.prefix + s, W) for s in range(w.decode_steps) for W in w.windows)
    fl_total = sum(attn_flops(w.B, w.n_q, w.d_h, w.prefix + s, 1, W)
                   for s in range(w.decode_steps) for W in w.windows)
    est = t_fixed + (t_attn / n) * (by_total / by_call)
    return {"value": round(by_total / est / 1e9, 3), "unit": "GB/s",
            "tflops": round(fl_total / est / 1e12, 6), "est_64_steps_s": round(est, 1),
            "sample": "fp64 numpy oracle on %s: %d timed decode queries (sequence 0, all heads, "
                      "full layer, %d allowed rows, %.2f s each) plus RoPE and the append "
                      "(%.2f s); all sequences, both layers and all %d steps extrapolated by "
                      "algorithmic bytes" % (w.name, n, p + 1, t_attn / n, t_fixed, w.decode_steps)}


def progress(what):
    """One line on stderr per finished phase (stdout holds only the JSON line)."""
    print("[bench] %s" % what, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl
    import long_context_sparse_yarn_amd as sa

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}))
        return
    if args.extra_only:
        leg = {"sampling": sample_extra, "moe": moe_extra, "qkv": qkv_extra}[args.extra_only]
        print(json.dumps({args.extra_only: leg(sa, torch)}), flush=True)
        return

    # ---- the headline: the handover workload
    w = wl.HANDOVER
    t = time_handover(w, sa, torch, args.steps, args.warmup, args.settle_ms)
    pre, dec = handover_flops(w)
    fl_step = sum(pre.values()) + sum(dec.values())
    value = fl_step / (t["ms_step"] * 1e-3) / 1e12
    ho = handover_figures(w, t)
    progress("handover timed: %.4f ms per step" % t["ms_step"])
    full = [f for f in ho["layers"] if f["window"] == 0][0]
    traffic = TRAFFIC.get(("handover", 0))
    roofline = {"bound": "mfma", "achieved": full["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": full["frac_mfma"],
                "traffic": (traffic["bytes"] if traffic and
                            kernel_sources_hash() == traffic["sources_sha256_16"] else None),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)",
                "kernel": prefill_kernel_name(w.d_h, False) + " (full causal)",
                "kernel_gflop": full["gflop"],
                "kernel_ms": full["kernel_ms"], "kernel_timing": full["kernel_timing"]}
    line = {
        "metric": "sink-GQA attention prefill TFLOP/s + decode KV GB/s, % of MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["ms_step"], 4),
        "step_spread": {"median_ms": round(float(np.median(t["per_step"])), 4),
                        "min_ms": round(float(np.min(t["per_step"])), 4),
                        "pass": "the same steps again after the timed region, an event at each "
                                "step boundary"},
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "global_batch": w.B, "prefix_rows": w.prefix,
                   "chunk": w.T, "decode_steps": "2 sweeps x %d (restore between)" % w.decode_steps,
                   "n_q": w.n_q, "n_kv": w.n_kv, "d_h": w.d_h, "windows": list(w.windows),
                   "yarn": {"base": w.yarn.base, "factor": w.yarn.factor,
                            "orig_ctx": w.yarn.orig_ctx}, "parallelism": "single GPU"},
        "settle": {"ms": args.settle_ms, "launches": t["settle_launches"],
                   "what": "back-to-back full-causal prefill launches before the warmup steps, "
                           "untimed, so the timed steps run at the clock this load holds"},
        "roofline": roofline,
        "handover": ho,
    }

    # ---- long-context decode: the second headline figure (KV GB/s)
    ld = decode_extra(sa, torch)
    fd = ld["full"]
    progress("long decode timed")
    line["decode_kv"] = {"workload": ld["workload"], "layer": "full causal",
                         "gbs": fd["gbs"], "frac_hbm": fd["frac_hbm"],
                         "attn_kernel_us": fd["attn_kernel_us"], "step_us": fd["step_us"],
                         "alg_mb_per_step": fd["alg_mb_per_step"], "peak_gbs": PEAK_HBM_GBS,
                         "timing": "events around each step's attention launches (split-KV kernel "
                                   "+ merge), 64 steps, queued behind a spin kernel so that the "
                                   "events time the GPU, not the host's calls"}
    cpu = {}
    if not args.no_extra:
        lw = wl.LITE_PREFILL
        layers, ms_step, kern_ms, in_step = time_prefill_step(lw, sa, torch, 20, 200)
        fl = sum(attn_flops(lw.B, lw.n_q, lw.d_h, lw.prefix, lw.T, L.window) for L in layers)
        per_layer = [prefill_figures(lw, L, kern_ms[i], in_step[i]) for i, L in enumerate(layers)]
        for i, p in IN_STEP_STATS.items():
            per_layer[i]["kernel_ms_in_step_median"] = round(p[0], 4)
            per_layer[i]["kernel_ms_in_step_min"] = round(p[1], 4)
        full_i = [i for i, L in enumerate(layers) if L.window == 0][0]
        line["extra"] = {"gpt_oss_lite_prefill": {
            "workload": lw.name, "ms_per_step": round(ms_step, 4),
            "tflops_step": round(fl / (ms_step * 1e-3) / 1e12, 1), "layers": per_layer,
            "abi_calls": abi_call_figures(lw, layers[full_i], sa, torch),
            "ring": ring_prefill_figures(lw, [L for L in layers if L.window > 0][0], sa, torch)}}
        progress("gpt-oss-lite prefill timed")
        if not args.no_cpu:
            cpu["gpt-oss-lite prefill"] = cpu_prefill_sample(lw, layers, args.cpu_seconds)
        del layers
        torch.cuda.empty_cache()
        g = wl.GPTOSS_PREFILL
        gl, gms, gk, gin = time_prefill_step(g, sa, torch, 20, 200)
        fl = sum(attn_flops(g.B, g.n_q, g.d_h, g.prefix, g.T, L.window) for L in gl)
        line["extra"]["gpt_oss_prefill"] = {"workload": g.name, "ms_per_step": round(gms, 4),
                                            "tflops_step": round(fl / (gms * 1e-3) / 1e12, 1),
                                            "layers": [prefill_figures(g, L, gk[i], gin[i])
                                                       for i, L in enumerate(gl)]}
        progress("gpt-oss prefill timed")
        if not args.no_cpu:
            cpu["gpt-oss prefill"] = cpu_prefill_sample(g, gl, args.cpu_seconds)
        del gl
        torch.cuda.empty_cache()
        line["extra"]["long_decode"] = ld
        line["extra"]["qkv_projection"] = qkv_extra(sa, torch)
        progress("projection timed")
        line["extra"]["moe_layer"] = moe_extra(sa, torch)
        progress("MoE layer timed")
        line["extra"]["sampling"] = sample_extra(sa, torch)
        progress("sampling timed")
    if not args.no_cpu:
        head = cpu_prefill_sample(w, t["layers"], 2 * args.cpu_seconds, extra_flops=dec)
        cores, model = _cpu_info()
        if not args.no_extra:
            cpu["long decode"] = cpu_decode_sample(wl.LONG_DECODE, args.cpu_seconds)
        line["cpu_baseline"] = {**head, "cores": cores, "cpu_model": model,
                                "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
                                "per_workload": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
