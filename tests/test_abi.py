"""C-ABI checks that need no GPU: the library loads, exports every function
include/sinkattn.h declares, its host logic (YaRN table, KV byte count,
snapshot bookkeeping) agrees with the oracle, and every argument error is
reported before anything is enqueued (no call here launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")

sa = pytest.importorskip("long_context_sparse_yarn_amd",
                         reason="libsinkattn.so not built (run __graft_entry__.build())")
from long_context_sparse_yarn_amd import _binding as B  # noqa: E402
from oracle.yarn import yarn_concentration, yarn_inv_freq  # noqa: E402

SA_OK, SA_ERR_ARG, SA_ERR_SHAPE, SA_ERR_DTYPE, SA_ERR_CAPACITY, SA_ERR_SNAPSHOT = 0, -1, -2, -3, -4, -5
FAKE_K, FAKE_V = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)   # never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s+\**\s*([A-Za-z_]\w*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("yarn_rope_apply", "kv_cache_append", "kv_cache_snapshot", "kv_cache_restore",
              "sinkattn_prefill", "sinkattn_decode"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.parametrize("d,base,s,L,a,b", [(64, 150000.0, 32.0, 4096, 1.0, 32.0),
                                            (96, 150000.0, 32.0, 4096, 1.0, 32.0),
                                            (64, 10000.0, 1.0, 4096, 1.0, 32.0),
                                            (128, 500000.0, 8.0, 8192, 2.0, 16.0)])
def test_host_yarn_table_matches_oracle(d, base, s, L, a, b):
    inv, c = sa.yarn_inv_freq(sa.Yarn(d, base, s, L, a, b))
    np.testing.assert_allclose(inv, yarn_inv_freq(d, base, s, L, a, b), rtol=4e-16, atol=0)
    assert c == pytest.approx(yarn_concentration(s), rel=1e-15)


def test_yarn_bad_parameters():
    with pytest.raises(sa.SinkAttnError):
        sa.yarn_inv_freq(sa.Yarn(64, 150000.0, 0.5))
    with pytest.raises(sa.SinkAttnError):
        sa.yarn_inv_freq(sa.Yarn(64, ntk_alpha=32.0, ntk_beta=1.0))


def test_kv_cache_bytes():
    assert sa.kv_cache_bytes(24, 1, 131072, 8, 64, 2) == 6442450944   # the printed 6.0 GiB
    assert sa.kv_cache_bytes(1, 8, 131136, 8, 64, 2) == 2 * 8 * 131136 * 8 * 64 * 2
    assert sa.kv_cache_bytes(1 << 40, 1 << 40, 2, 2, 2, 2) == -1
    assert sa.kv_cache_bytes(-1, 1, 1, 1, 1, 1) == -1


def create(dtype=0, Bn=2, C=256, n_kv=2, d=64, offset=0):
    h = ctypes.c_void_p()
    st = B._kv_cache_create(ctypes.byref(h), FAKE_K, FAKE_V, dtype, Bn, C, n_kv, d, offset)
    return st, h


def test_cache_create_validation():
    assert create(C=100)[0] == SA_ERR_SHAPE          # not a multiple of 32
    assert create(C=0)[0] == SA_ERR_SHAPE
    assert create(dtype=7)[0] == SA_ERR_DTYPE
    assert create(d=60)[0] == SA_ERR_SHAPE
    assert create(offset=300)[0] == SA_ERR_CAPACITY
    h = ctypes.c_void_p()
    assert B._kv_cache_create(ctypes.byref(h), None, FAKE_V, 0, 2, 256, 2, 64, 0) == SA_ERR_ARG
    assert "null" in sa.last_error()
    h2 = ctypes.c_void_p()
    assert B._kv_cache_create(ctypes.byref(h2), ctypes.c_void_p(0x10008), FAKE_V, 0, 2, 256, 2,
                              64, 0) == SA_ERR_ARG                      # not 16-byte aligned
    st, h = create(offset=40)
    assert st == SA_OK and B._kv_cache_offset(h) == 40
    assert B._kv_cache_offset(None) == -1
    assert B._kv_cache_destroy(h) == SA_OK
    assert B._kv_cache_destroy(None) == SA_ERR_ARG
    # kv_cache_init: the constructor under the cache interface's own name
    lib = ctypes.CDLL(B.LIB_PATH)
    init = lib.kv_cache_init
    init.restype = ctypes.c_int
    init.argtypes = B._kv_cache_create.argtypes
    hi = ctypes.c_void_p()
    assert init(ctypes.byref(hi), FAKE_K, FAKE_V, 0, 2, 256, 2, 64, 17) == SA_OK
    assert B._kv_cache_offset(hi) == 17 and B._kv_cache_base(hi) == 0
    assert init(ctypes.byref(ctypes.c_void_p()), FAKE_K, FAKE_V, 0, 2, 100, 2, 64, 0) == SA_ERR_SHAPE
    assert B._kv_cache_destroy(hi) == SA_OK


def test_errors_are_reported_before_any_launch():
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=10)
    assert st == SA_OK
    q, o, s = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000)
    # append past capacity
    assert B._kv_cache_append(h, q, q, 247, None) == SA_ERR_CAPACITY
    assert B._kv_cache_append(h, q, q, 0, None) == SA_ERR_ARG
    assert B._kv_cache_offset(h) == 10                                    # unchanged
    # prefill: queries past the rows in the cache; GQA contract; head dim
    P = B._sinkattn_prefill
    assert P(q, h, s, o, 2, 5, 8, 2, 64, 0, 0.125, 6, None) == SA_ERR_CAPACITY
    assert P(q, h, s, o, 2, 5, 7, 2, 64, 0, 0.125, 0, None) == SA_ERR_SHAPE
    assert P(q, h, s, o, 2, 5, 8, 4, 64, 0, 0.125, 0, None) == SA_ERR_SHAPE   # n_kv != cache
    assert P(q, h, s, o, 3, 5, 8, 2, 64, 0, 0.125, 0, None) == SA_ERR_SHAPE   # B != cache
    assert P(q, h, s, o, 2, 5, 8, 2, 64, 0, 0.0, 0, None) == SA_ERR_ARG
    assert P(None, h, s, o, 2, 5, 8, 2, 64, 0, 0.125, 0, None) == SA_ERR_ARG
    assert P(ctypes.c_void_p(0x30004), h, s, o, 2, 5, 8, 2, 64, 0, 0.125, 0, None) == SA_ERR_ARG
    assert P(q, h, s, o, 2, 0, 8, 2, 64, 0, 0.125, 0, None) == SA_OK          # nothing to do
    # decode: q_mult > 16 on bf16, workspace too small
    D = B._sinkattn_decode
    assert D(q, h, s, o, 2, 64, 2, 64, 0, 0.125, o, 1 << 30, None) == SA_ERR_SHAPE
    need = B._sinkattn_decode_ws(2, 8, 2, 64, 256)
    assert need > 0
    assert D(q, h, s, o, 2, 8, 2, 64, 0, 0.125, o, need - 4, None) == SA_ERR_ARG
    assert D(q, h, s, o, 2, 8, 2, 64, 0, 0.125, None, need, None) == SA_ERR_ARG
    B._kv_cache_destroy(h)
    # bf16 attention head dims
    st, h80 = create(d=80, offset=10)
    assert st == SA_OK
    assert P(q, h80, s, o, 2, 5, 8, 2, 80, 0, 0.125, 0, None) == SA_ERR_SHAPE
    B._kv_cache_destroy(h80)
    # bf16 prefill keeps key positions in 32 bits: a 2^31-row cache is refused
    st, hbig = create(Bn=1, C=(1 << 31), n_kv=2, d=64, offset=10)
    assert st == SA_OK
    assert P(q, hbig, s, o, 1, 5, 8, 2, 64, 0, 0.125, 0, None) == SA_ERR_SHAPE
    assert "2^31" in sa.last_error()
    # so does bf16 decode (its block indices are 32-bit)
    assert D(q, hbig, s, o, 1, 8, 2, 64, 0, 0.125, o, 1 << 20, None) == SA_ERR_SHAPE
    assert "2^31" in sa.last_error()
    B._kv_cache_destroy(hbig)
    # prefill with in-kernel rotation: yarn checks and bf16 only, nothing launched
    PR = B._sinkattn_prefill_rope
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=10)
    yq = B.SaYarn(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    yq96 = B.SaYarn(96, 150000.0, 32.0, 4096, 1.0, 32.0)
    assert PR(q, h, s, o, 2, 5, 8, 2, 64, 0, 0.125, 0, None, None) == SA_ERR_ARG
    assert PR(q, h, s, o, 2, 5, 8, 2, 64, 0, 0.125, 0, ctypes.byref(yq96), None) == SA_ERR_SHAPE
    assert PR(q, h, s, o, 2, 5, 8, 2, 64, 0, 0.125, 6, ctypes.byref(yq), None) == SA_ERR_CAPACITY
    assert PR(q, h, s, o, 2, 0, 8, 2, 64, 0, 0.125, 0, ctypes.byref(yq), None) == SA_OK
    B._kv_cache_destroy(h)
    st, hf = create(dtype=1, Bn=2, C=256, n_kv=2, d=64, offset=10)
    assert PR(q, hf, s, o, 2, 5, 8, 2, 64, 0, 0.125, 0, ctypes.byref(yq), None) == SA_ERR_DTYPE
    B._kv_cache_destroy(hf)
    # rotate-and-append: yarn checks, bf16 head dim, capacity, nothing launched
    AR = B._kv_cache_append_rope
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=10)
    y64 = B.SaYarn(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    y96 = B.SaYarn(96, 150000.0, 32.0, 4096, 1.0, 32.0)
    assert AR(h, q, q, 4, None, None) == SA_ERR_ARG                         # no yarn
    assert AR(h, q, q, 4, ctypes.byref(y96), None) == SA_ERR_SHAPE           # yarn d_h differs
    assert AR(h, q, q, 247, ctypes.byref(y64), None) == SA_ERR_CAPACITY
    assert AR(h, ctypes.c_void_p(0x30008), q, 4, ctypes.byref(y64), None) == SA_ERR_ARG
    assert B._kv_cache_offset(h) == 10
    B._kv_cache_destroy(h)
    # with queries: both or neither, aligned, n_q > 0, no partial overlap
    QK = B._kv_cache_append_rope_qk
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=10)
    qr = ctypes.c_void_p(0x60000)
    assert QK(h, q, None, 8, q, q, 4, ctypes.byref(y64), None) == SA_ERR_ARG
    assert QK(h, q, ctypes.c_void_p(0x60008), 8, q, q, 4, ctypes.byref(y64), None) == SA_ERR_ARG
    assert QK(h, q, qr, 0, q, q, 4, ctypes.byref(y64), None) == SA_ERR_ARG
    assert QK(h, q, ctypes.c_void_p(0x30000 + 128), 8, q, q, 4, ctypes.byref(y64), None) == SA_ERR_ARG
    assert QK(h, q, qr, 8, q, q, 4, ctypes.byref(y96), None) == SA_ERR_SHAPE
    assert B._kv_cache_offset(h) == 10
    B._kv_cache_destroy(h)
    st, h24 = create(d=24, offset=10)
    y24 = B.SaYarn(24, 150000.0, 32.0, 4096, 1.0, 32.0)
    assert AR(h24, q, q, 4, ctypes.byref(y24), None) == SA_ERR_SHAPE         # bf16 needs d % 16
    B._kv_cache_destroy(h24)
    # rope
    y = B.SaYarn(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    R = B._yarn_rope_apply
    assert R(q, 9, 1, 4, 8, 64, 0, ctypes.byref(y), None) == SA_ERR_DTYPE
    assert R(q, 0, 1, 4, 8, 60, 0, ctypes.byref(y), None) == SA_ERR_SHAPE
    assert R(q, 0, 1, 4, 8, 96, 0, ctypes.byref(y), None) == SA_ERR_SHAPE   # yarn d_h 64
    assert R(q, 0, 1, 4, 8, 64, -1, ctypes.byref(y), None) == SA_ERR_ARG
    assert R(q, 0, 1, 0, 8, 64, 0, ctypes.byref(y), None) == SA_OK          # T = 0
    R2 = B._yarn_rope
    # out of place: partial overlap refused, exact aliasing allowed (no launch at T = 0)
    assert R2(q, ctypes.c_void_p(0x30000 + 64), 0, 1, 4, 8, 64, 0, ctypes.byref(y), None) == SA_ERR_ARG
    assert R2(q, q, 0, 1, 0, 8, 64, 0, ctypes.byref(y), None) == SA_OK


def test_snapshot_bookkeeping_without_appends():
    st, h = create(offset=64)
    st2, other = create(offset=64)
    snap = B.SaSnapshot()
    assert B._kv_cache_snapshot(h, ctypes.byref(snap)) == SA_OK
    assert snap.offset == 64
    assert B._kv_cache_restore(other, ctypes.byref(snap)) == SA_ERR_SNAPSHOT   # foreign
    assert B._kv_cache_restore(h, ctypes.byref(snap)) == SA_OK
    bad = B.SaSnapshot(64, snap.cache_id, snap.stamp + 5)                      # from the future
    assert B._kv_cache_restore(h, ctypes.byref(bad)) == SA_ERR_SNAPSHOT
    B._kv_cache_destroy(h)
    B._kv_cache_destroy(other)


def test_decode_workspace_size_bound():
    # grows with capacity until the split cap, never zero for valid shapes
    a = B._sinkattn_decode_ws(8, 64, 8, 64, 131136)
    b = B._sinkattn_decode_ws(8, 64, 8, 64, 256)
    assert a >= b > 0
    assert B._sinkattn_decode_ws(8, 63, 8, 64, 256) == 0


def test_binding_counts_workspace_bytes_of_any_dtype():
    """The binding hands the C-ABI the workspace's size in bytes whatever its
    dtype, so a too-small workspace of a narrow dtype is refused by the
    library's size check instead of being written past its end."""
    import torch
    need = B._sinkattn_decode_ws(2, 8, 2, 64, 256)
    for dt in (torch.float32, torch.bfloat16, torch.uint8, torch.int64):
        esz = torch.tensor([], dtype=dt).element_size()
        small = torch.empty((need - 1) // esz, dtype=dt)          # one element short of `need`
        assert B._nbytes(small) == small.numel() * esz < need
        big = torch.empty((need + esz - 1) // esz, dtype=dt)
        assert B._nbytes(big) >= need
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=10)
    q, o, s = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000)
    small = torch.empty((need - 1) // 2, dtype=torch.bfloat16)
    assert B._sinkattn_decode(q, h, s, o, 2, 8, 2, 64, 0, 0.125, o, B._nbytes(small),
                              None) == SA_ERR_ARG
    B._kv_cache_destroy(h)


def test_binding_checks_out_before_any_launch():
    import torch
    q = torch.empty((2, 5, 8, 64), dtype=torch.bfloat16)
    assert B._out_like(q, None).shape == q.shape
    good = torch.empty_like(q)
    assert B._out_like(q, good) is good
    for bad in (torch.empty((2, 5, 8, 32), dtype=torch.bfloat16),        # shape
                torch.empty((2, 5, 8, 64), dtype=torch.float32),         # dtype
                torch.empty((2, 5, 64, 8), dtype=torch.bfloat16).transpose(2, 3)):  # layout
        with pytest.raises(ValueError):
            B._out_like(q, bad)


def test_noalloc_decode_refuses_what_its_scratch_cannot_hold():
    """sinkattn_decode_noalloc checks its partials' size against the static
    scratch before it touches the device: B 8, 128 query heads over 8 KV
    heads at d 128 on a 2000-row span need 17 MB of partials."""
    assert B._sinkattn_decode_scratch_bytes() == 8 << 20
    st, h = create(Bn=8, C=2048, n_kv=8, d=128, offset=2000)
    assert st == SA_OK
    q, o, s = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000)
    assert B._sinkattn_decode_noalloc(q, h, s, o, 8, 128, 8, 128, 0, 0.125, None) == SA_ERR_ARG
    assert "static scratch" in sa.last_error()
    # argument errors come first, as in sinkattn_decode
    assert B._sinkattn_decode_noalloc(None, h, s, o, 8, 128, 8, 128, 0, 0.125, None) == SA_ERR_ARG
    assert B._sinkattn_decode_noalloc(q, h, s, o, 8, 127, 8, 128, 0, 0.125, None) == SA_ERR_SHAPE
    B._kv_cache_destroy(h)


def test_decode_step_checks_before_enqueueing():
    """sinkattn_decode_step runs the append's and the decode's checks before
    it enqueues anything, and leaves the offset alone on every error."""
    ys = B.Yarn(64).c_struct()
    yp = ctypes.byref(ys)
    q, qr, o, s = (ctypes.c_void_p(a) for a in (0x30000, 0x60000, 0x40000, 0x50000))
    k, v, ws = ctypes.c_void_p(0x70000), ctypes.c_void_p(0x80000), ctypes.c_void_p(0x90000)
    step = B._sinkattn_decode_step
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=255)
    assert st == SA_OK
    args = lambda **kw: [kw.get("c", h), kw.get("q", q), kw.get("qr", qr), kw.get("k", k),
                         kw.get("v", v), s, kw.get("o", o), 2, kw.get("n_q", 8), 2, 64,
                         kw.get("W", 0), 0.125, kw.get("y", yp), ws, 1 << 20, None]
    assert step(*args(k=None)) == SA_ERR_ARG
    assert step(*args(q=None)) == SA_ERR_ARG
    assert step(*args(y=None)) == SA_ERR_ARG
    assert step(*args(qr=ctypes.c_void_p(0x30000 + 64))) == SA_ERR_ARG      # q_rot overlaps q
    assert "overlaps" in sa.last_error()
    assert step(*args(qr=ctypes.c_void_p(0x40000))) == SA_ERR_ARG           # q_rot is out
    assert step(*args(qr=ctypes.c_void_p(0x60008))) == SA_ERR_ARG           # misaligned
    assert step(*args(n_q=7)) == SA_ERR_SHAPE                               # 7 heads over 2 KV heads
    assert step(*args(n_q=40)) == SA_ERR_SHAPE                              # q_mult 20 > 16
    assert B._kv_cache_offset(h) == 255
    B._kv_cache_destroy(h)
    # a full cache: the append's capacity check
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=256)
    assert step(*args(c=h)) == SA_ERR_CAPACITY
    assert B._kv_cache_offset(h) == 256
    B._kv_cache_destroy(h)
    # fp32 caches attend through the separate calls
    st, h = create(dtype=1, Bn=2, C=256, n_kv=2, d=64, offset=3)
    assert step(*args(c=h)) == SA_ERR_DTYPE
    assert B._kv_cache_offset(h) == 3
    B._kv_cache_destroy(h)
    # a ring takes window == W only
    st, r = ring()
    assert step(*args(c=r, W=64)) == SA_ERR_ARG
    assert B._kv_cache_offset(r) == 0
    B._kv_cache_destroy(r)


def ring(dtype=0, Bn=2, W=128, n_kv=2, d=64):
    h = ctypes.c_void_p()
    st = B._kv_ring_create(ctypes.byref(h), FAKE_K, FAKE_V, dtype, Bn, W, n_kv, d)
    return st, h


def test_ring_create_and_host_bookkeeping():
    assert ring(W=100)[0] == SA_ERR_SHAPE                 # window not a multiple of 32
    assert ring(W=0)[0] == SA_ERR_SHAPE
    assert ring(dtype=5)[0] == SA_ERR_DTYPE
    st, r = ring()
    assert st == SA_OK
    assert B._kv_cache_offset(r) == 0 and B._kv_cache_base(r) == 0
    st, lin = create(Bn=2, C=256, n_kv=2, d=64, offset=0)
    q, o, s = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000)
    # a ring is never attended by prefill; decode needs the step's row first
    P = B._sinkattn_prefill
    assert P(q, r, s, o, 2, 1, 8, 2, 64, 128, 0.125, 0, None) == SA_ERR_ARG
    assert "stage" in sa.last_error()
    assert B._sinkattn_decode(q, r, s, o, 2, 8, 2, 64, 128, 0.125, o, 1 << 20, None) == SA_ERR_CAPACITY
    # staging: direction, shapes and dtype checked; an empty ring stages nothing
    ST, CM = B._kv_ring_stage, B._kv_ring_commit
    assert ST(r, lin, None) == SA_ERR_ARG                 # arguments swapped
    st, r2 = ring()
    assert ST(r2, r, None) == SA_ERR_ARG                  # stage must be linear
    st, lin3 = create(Bn=2, C=256, n_kv=2, d=96)
    assert ST(lin3, r, None) == SA_ERR_SHAPE
    st, linf = create(dtype=1, Bn=2, C=256, n_kv=2, d=64)
    assert ST(linf, r, None) == SA_ERR_DTYPE
    assert CM(r, lin, None) == SA_ERR_SNAPSHOT            # never staged from r
    assert ST(lin, r, None) == SA_OK                      # nothing to copy: no launch
    assert B._kv_cache_offset(lin) == 0 and B._kv_cache_base(lin) == 0
    assert CM(r2, lin, None) == SA_ERR_SNAPSHOT           # staged from another ring
    assert CM(r, lin, None) == SA_OK                      # nothing new: no launch
    assert CM(r, lin, None) == SA_OK                      # re-commit after commit is fine
    # save/load: argument checks before any copy
    snap = B.SaSnapshot()
    ks, vs = ctypes.c_void_p(0x70000), ctypes.c_void_p(0x80000)
    assert B._kv_ring_save(lin, ks, vs, ctypes.byref(snap), None) == SA_ERR_ARG   # not a ring
    assert B._kv_ring_save(r, None, vs, ctypes.byref(snap), None) == SA_ERR_ARG
    assert B._kv_ring_save(r, ctypes.c_void_p(0x70008), vs, ctypes.byref(snap), None) == SA_ERR_ARG
    assert B._kv_cache_snapshot(r2, ctypes.byref(snap)) == SA_OK
    assert B._kv_ring_load(r, ks, vs, ctypes.byref(snap), None) == SA_ERR_SNAPSHOT  # foreign
    assert B._kv_ring_load(lin, ks, vs, ctypes.byref(snap), None) == SA_ERR_ARG
    # O(1) restore of a ring with nothing appended since the snapshot is allowed
    assert B._kv_cache_snapshot(r, ctypes.byref(snap)) == SA_OK
    assert B._kv_cache_restore(r, ctypes.byref(snap)) == SA_OK
    for h in (r, r2, lin, lin3, linf):
        B._kv_cache_destroy(h)


def test_qkv_errors_before_any_launch():
    Q = B._sinkattn_qkv
    y64 = B.SaYarn(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    x, w, b, q, ws = (ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000),
                      ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000))
    need = B._sinkattn_qkv_ws(100, 64)
    assert need == 100 * 32 * 16
    st, h = create(Bn=2, C=256, n_kv=2, d=64, offset=10)
    args = lambda **k: dict(dict(c=h, x=x, w=w, b=b, q=q, B=2, T=100, dm=128, n_q=8, y=ctypes.byref(y64),
                                 ws=ws, wsb=need), **k)
    call = lambda a: Q(a["c"], a["x"], a["w"], a["b"], a["q"], a["B"], a["T"], a["dm"], a["n_q"], a["y"],
                       a["ws"], a["wsb"], None)
    assert call(args(x=None)) == SA_ERR_ARG
    assert call(args(x=ctypes.c_void_p(0x30008))) == SA_ERR_ARG            # misaligned
    assert call(args(dm=100)) == SA_ERR_SHAPE                                # d_model % 64
    assert call(args(B=3)) == SA_ERR_SHAPE                                   # B != cache
    assert call(args(T=247)) == SA_ERR_CAPACITY                              # 10 + 247 > 256
    assert call(args(wsb=need - 16)) == SA_ERR_ARG
    assert call(args(T=0)) == SA_ERR_ARG
    y96 = B.SaYarn(96, 150000.0, 32.0, 4096, 1.0, 32.0)
    assert call(args(y=ctypes.byref(y96))) == SA_ERR_SHAPE                   # yarn d_h differs
    assert B._kv_cache_offset(h) == 10
    B._kv_cache_destroy(h)
    st, hf = create(dtype=1, Bn=2, C=256, n_kv=2, d=64)
    assert call(args(c=hf)) == SA_ERR_DTYPE
    B._kv_cache_destroy(hf)
    st, h80 = create(Bn=2, C=256, n_kv=2, d=80)
    assert call(args(c=h80)) == SA_ERR_SHAPE
    B._kv_cache_destroy(h80)
    st, r = ring(Bn=2, W=128, n_kv=2, d=64)
    assert call(args(c=r)) == SA_ERR_ARG                                     # a ring: use its stage
    B._kv_cache_destroy(r)


def test_moe_errors_before_any_launch():
    x, w, y, ws = (ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000),
                   ctypes.c_void_p(0x60000))
    ids, wt, lg = ctypes.c_void_p(0x70000), ctypes.c_void_p(0x80000), ctypes.c_void_p(0x90000)
    R = B._moe_route
    assert R(x, 100, 64, w, 65, 2, lg, ids, wt, None) == SA_ERR_SHAPE        # E > 64
    assert R(x, 100, 64, w, 8, 9, lg, ids, wt, None) == SA_ERR_SHAPE         # k > 8
    assert R(x, 100, 64, w, 2, 3, lg, ids, wt, None) == SA_ERR_SHAPE         # k > E
    assert R(x, 100, 96, w, 8, 2, lg, ids, wt, None) == SA_ERR_SHAPE         # d_model % 64
    assert R(None, 100, 64, w, 8, 2, lg, ids, wt, None) == SA_ERR_ARG
    assert R(x, 0, 64, w, 8, 2, lg, ids, wt, None) == SA_ERR_ARG
    D = B._moe_dispatch
    need = B._moe_dispatch_ws(1000, 8)
    assert need > 0
    assert D(ids, 1000, 8, 2, y, y, ws, need - 1, None) == SA_ERR_ARG
    assert D(ids, 1000, 65, 2, y, y, ws, need, None) == SA_ERR_SHAPE
    L = B._moe_layer
    nb = B._moe_ws(100, 64, 8, 2, 128, 0)
    assert nb > 0 and B._moe_ws(100, 64, 8, 2, 128, 128) > nb
    assert L(x, 100, 64, w, 8, 2, w, w, 100, None, None, 0, y, ws, nb, None) == SA_ERR_SHAPE   # ffn % 128
    assert L(x, 100, 64, w, 8, 2, w, w, 128, None, None, 0, y, ws, nb - 1, None) == SA_ERR_ARG
    assert L(x, 100, 64, w, 8, 2, w, w, 128, w, None, 128, y, ws, 1 << 30, None) == SA_ERR_ARG  # half the shared
    assert L(x, 100, 64, w, 8, 2, w, w, 128, w, w, 0, y, ws, 1 << 30, None) == SA_ERR_ARG       # weights, no ffn
    assert L(x, 100, 64, w, 8, 2, w, w, 128, None, None, 0, ctypes.c_void_p(0x50004), ws, nb,
             None) == SA_ERR_ARG


def test_sample_errors_before_any_launch():
    lg, pr, u, tok, ws = (ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000),
                          ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000))
    cnt = ctypes.c_void_p(0x80000)
    assert ctypes.sizeof(B.SaSampleParams) == 32
    need = B._sample_ws(8, 128000)
    assert need >= 8 * 128000 * 4 and B._sample_ws(8, 262145) == 0 and B._sample_ws(0, 10) == 0
    S = B._sample_tokens

    def call(B_=8, V=128000, ls=128000, bias=None, bs=0, counts=None, upd=0, ws_=ws, nb=need, **kw):
        return S(kw.get("logits", lg), B_, V, ls, bias, bs, counts, kw.get("params", pr), kw.get("u", u),
                 upd, kw.get("tokens", tok), None, None, ws_, nb, None)

    assert call(V=0) == SA_ERR_SHAPE
    assert call(V=262145, ls=262145) == SA_ERR_SHAPE
    assert call(B_=0) == SA_ERR_SHAPE
    assert call(B_=65536) == SA_ERR_SHAPE
    assert call(ls=127999) == SA_ERR_ARG                     # row stride below V
    assert call(bias=lg, bs=5) == SA_ERR_ARG                 # bias stride neither 0 nor >= V
    assert call(upd=1) == SA_ERR_ARG                         # update without counts
    assert call(nb=need - 1) == SA_ERR_ARG
    assert call(ws_=ctypes.c_void_p(0x70008)) == SA_ERR_ARG  # misaligned workspace
    assert call(logits=None) == SA_ERR_ARG
    assert call(params=None) == SA_ERR_ARG
    assert call(u=None) == SA_ERR_ARG
    assert call(tokens=None) == SA_ERR_ARG
    C = B._sample_count_tokens
    assert C(lg, 8, 10, 9, cnt, 100, None) == SA_ERR_ARG     # stride below H
    assert C(lg, 8, -1, 9, cnt, 100, None) == SA_ERR_ARG
    assert C(lg, 8, 10, 10, None, 100, None) == SA_ERR_ARG
    assert C(lg, 8, 10, 10, cnt, 0, None) == SA_ERR_SHAPE
    assert C(None, 8, 0, 0, cnt, 100, None) == SA_OK         # nothing to count: no launch
