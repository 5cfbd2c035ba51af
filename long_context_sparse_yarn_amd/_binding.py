"""ctypes binding over libsinkattn.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into device pointers, torch's current stream into the HIP
stream argument, and non-OK statuses into exceptions.  It loads the library
at import and fails loudly when it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsinkattn.so")

SA_BF16, SA_F32 = 0, 1
STATUS = {0: "SA_OK", -1: "SA_ERR_ARG", -2: "SA_ERR_SHAPE", -3: "SA_ERR_DTYPE",
          -4: "SA_ERR_CAPACITY", -5: "SA_ERR_SNAPSHOT", -6: "SA_ERR_HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libsinkattn.so is not built (%s); run `python long_context_sparse_yarn_amd/build.py` "
        "or __graft_entry__.build()" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _u64, _f32, _f64 = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                ctypes.c_float, ctypes.c_double)
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t


class SaYarn(ctypes.Structure):
    _fields_ = [("d_h", ctypes.c_int32), ("base", _f64), ("factor", _f64),
                ("orig_ctx", _i64), ("ntk_alpha", _f64), ("ntk_beta", _f64)]


class SaSampleParams(ctypes.Structure):
    _fields_ = [("temperature", _f32), ("top_k", ctypes.c_int32), ("top_p", _f32), ("min_p", _f32),
                ("repetition", _f32), ("presence", _f32), ("frequency", _f32),
                ("reserved", ctypes.c_int32)]


class SaSnapshot(ctypes.Structure):
    _fields_ = [("offset", _i64), ("cache_id", _u64), ("stamp", _u64)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sa_last_error = _sig("sa_last_error", ctypes.c_char_p)
_sa_yarn_inv_freq = _sig("sa_yarn_inv_freq", _i32, ctypes.POINTER(SaYarn),
                         ctypes.POINTER(_f64), ctypes.POINTER(_f64))
_sa_kv_cache_bytes = _sig("sa_kv_cache_bytes", _i64, _i64, _i64, _i64, _i64, _i64, _i64)
_yarn_rope_apply = _sig("yarn_rope_apply", _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                        ctypes.POINTER(SaYarn), _vp)
_yarn_rope = _sig("yarn_rope", _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                  ctypes.POINTER(SaYarn), _vp)
_kv_cache_create = _sig("kv_cache_create", _i32, ctypes.POINTER(_vp), _vp, _vp, _i32, _i32,
                        _i64, _i32, _i32, _i64)
_kv_cache_destroy = _sig("kv_cache_destroy", _i32, _vp)
_kv_cache_offset = _sig("kv_cache_offset", _i64, _vp)
_kv_cache_base = _sig("kv_cache_base", _i64, _vp)
_kv_ring_create = _sig("kv_ring_create", _i32, ctypes.POINTER(_vp), _vp, _vp, _i32, _i32, _i32,
                       _i32, _i32)
_kv_ring_stage = _sig("kv_ring_stage", _i32, _vp, _vp, _vp)
_kv_ring_commit = _sig("kv_ring_commit", _i32, _vp, _vp, _vp)
_kv_ring_save = _sig("kv_ring_save", _i32, _vp, _vp, _vp, ctypes.POINTER(SaSnapshot), _vp)
_kv_ring_load = _sig("kv_ring_load", _i32, _vp, _vp, _vp, ctypes.POINTER(SaSnapshot), _vp)
_kv_cache_append = _sig("kv_cache_append", _i32, _vp, _vp, _vp, _i32, _vp)
_kv_cache_append_rope = _sig("kv_cache_append_rope", _i32, _vp, _vp, _vp, _i32,
                             ctypes.POINTER(SaYarn), _vp)
_kv_cache_append_rope_qk = _sig("kv_cache_append_rope_qk", _i32, _vp, _vp, _vp, _i32, _vp, _vp,
                                _i32, ctypes.POINTER(SaYarn), _vp)
_kv_cache_snapshot = _sig("kv_cache_snapshot", _i32, _vp, ctypes.POINTER(SaSnapshot))
_kv_cache_restore = _sig("kv_cache_restore", _i32, _vp, ctypes.POINTER(SaSnapshot))
_sinkattn_prefill = _sig("sinkattn_prefill", _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                         _i32, _i32, _f32, _i64, _vp)
_sinkattn_prefill_rope = _sig("sinkattn_prefill_rope", _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                              _i32, _i32, _i32, _i32, _f32, _i64, ctypes.POINTER(SaYarn), _vp)
_sinkattn_qkv_ws = _sig("sinkattn_qkv_workspace_bytes", _sz, _i32, _i32)
_sinkattn_qkv = _sig("sinkattn_qkv_rope_append", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                     _i32, ctypes.POINTER(SaYarn), _vp, _sz, _vp)
_moe_route = _sig("moe_route", _i32, _vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp)
_moe_dispatch_ws = _sig("moe_dispatch_workspace_bytes", _sz, _i32, _i32)
_moe_dispatch = _sig("moe_dispatch", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp)
_moe_ws = _sig("moe_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i32, _i32)
_moe_layer = _sig("moe_layer", _i32, _vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _vp,
                  _i32, _vp, _vp, _sz, _vp)
_sample_count_tokens = _sig("sample_count_tokens", _i32, _vp, _i32, _i32, _i64, _vp, _i32, _vp)
_sample_ws = _sig("sample_workspace_bytes", _sz, _i32, _i32)
_sample_tokens = _sig("sample_tokens", _i32, _vp, _i32, _i32, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _vp,
                      _vp, _vp, _vp, _sz, _vp)
_sinkattn_decode_ws = _sig("sinkattn_decode_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i64)
_sinkattn_decode = _sig("sinkattn_decode", _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                        _i32, _f32, _vp, _sz, _vp)
_sinkattn_decode_noalloc = _sig("sinkattn_decode_noalloc", _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                _i32, _i32, _i32, _f32, _vp)
_sinkattn_decode_scratch_bytes = _sig("sinkattn_decode_scratch_bytes", _sz)
_sinkattn_decode_step = _sig("sinkattn_decode_step", _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i32, _i32, _i32, _i32, _i32, _f32, ctypes.POINTER(SaYarn), _vp, _sz,
                             _vp)


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


def last_error() -> str:
    return (_sa_last_error() or b"").decode()


def _check(st: int) -> None:
    if st != 0:
        raise SinkAttnError(st, last_error())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    """Bytes a workspace tensor holds, whatever its dtype."""
    return t.numel() * t.element_size()


def _out_like(q: torch.Tensor, out: Optional[torch.Tensor]) -> torch.Tensor:
    """`out` if it can receive a result shaped like q, else a new tensor.
    A given `out` must match q's shape, dtype and device and be contiguous."""
    if out is None:
        return torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must match q in shape, dtype and device (%s %s %s vs %s %s %s)" % (
            tuple(out.shape), out.dtype, out.device, tuple(q.shape), q.dtype, q.device))
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    return out


@dataclass(frozen=True)
class Yarn:
    d_h: int
    base: float = 150000.0
    factor: float = 32.0
    orig_ctx: int = 4096
    ntk_alpha: float = 1.0
    ntk_beta: float = 32.0

    def c_struct(self) -> SaYarn:
        return SaYarn(self.d_h, self.base, self.factor, self.orig_ctx, self.ntk_alpha,
                      self.ntk_beta)


def yarn_inv_freq(y: Yarn):
    """Host table: (inv_freq list of d_h/2 floats, concentration)."""
    arr = (_f64 * (y.d_h // 2))()
    c = _f64()
    s = y.c_struct()
    _check(_sa_yarn_inv_freq(ctypes.byref(s), arr, ctypes.byref(c)))
    return list(arr), c.value


def kv_cache_bytes(L, B, T, H_kv, d, dtype_bytes) -> int:
    return int(_sa_kv_cache_bytes(L, B, T, H_kv, d, dtype_bytes))


def yarn_rope_apply(x: torch.Tensor, offset: int, y: Yarn, stream=None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rotate x [B, T, H, d] at positions offset + t: in place, or into `out`
    (same shape and dtype) when given.  Returns the rotated tensor."""
    if x.dim() != 4:
        raise ValueError("x must be [B, T, H, d]")
    B, T, H, d = x.shape
    s = y.c_struct()
    if out is None:
        _check(_yarn_rope_apply(_dev(x, "x"), _dtype_code(x), B, T, H, d, int(offset),
                                ctypes.byref(s), _stream(stream)))
        return x
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _check(_yarn_rope(_dev(x, "x"), _dev(out, "out"), _dtype_code(x), B, T, H, d, int(offset),
                      ctypes.byref(s), _stream(stream)))
    return out


def v_cache_shape(B: int, C: int, n_kv: int, d: int):
    """Shape of the blocked V buffer: [B, C/32, n_kv, d, 32]."""
    return (B, C // 32, n_kv, d, 32)


def v_rows(v_buf: torch.Tensor) -> torch.Tensor:
    """View a blocked V buffer [B, C/32, n_kv, d, 32] as rows [B, C, n_kv, d]."""
    B, nb, n_kv, d, w = v_buf.shape
    return v_buf.permute(0, 1, 4, 2, 3).reshape(B, nb * w, n_kv, d)


def v_blocked(v_rows_t: torch.Tensor) -> torch.Tensor:
    """Rows [B, C, n_kv, d] -> blocked layout [B, C/32, n_kv, d, 32] (a copy)."""
    B, C, n_kv, d = v_rows_t.shape
    return v_rows_t.reshape(B, C // 32, 32, n_kv, d).permute(0, 1, 3, 4, 2).contiguous()


class KVCache:
    """One layer's cache over caller-owned buffers k [B,C,n_kv,d] and
    v [B,C/32,n_kv,d,32] (see v_cache_shape)."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, offset: int = 0):
        if k.dim() != 4 or v.dim() != 5:
            raise ValueError("k must be [B,C,n_kv,d], v [B,C/32,n_kv,d,32]")
        B, C, n_kv, d = k.shape
        if tuple(v.shape) != v_cache_shape(B, C, n_kv, d) or v.dtype != k.dtype:
            raise ValueError("v buffer shape/dtype does not match k")
        self.k, self.v = k, v
        self.B, self.capacity, self.n_kv, self.d = B, C, n_kv, d
        self.dtype = k.dtype
        h = _vp()
        _check(_kv_cache_create(ctypes.byref(h), _dev(k, "k"), _dev(v, "v"), _dtype_code(k),
                                B, C, n_kv, d, int(offset)))
        self._h = h

    @classmethod
    def empty(cls, B, C, n_kv, d, dtype=torch.bfloat16, device="cuda", fill=None):
        k = torch.empty((B, C, n_kv, d), dtype=dtype, device=device)
        v = torch.empty(v_cache_shape(B, C, n_kv, d), dtype=dtype, device=device)
        if fill is not None:
            k.fill_(fill)
            v.fill_(fill)
        return cls(k, v)

    @property
    def handle(self):
        return self._h

    @property
    def offset(self) -> int:
        """Positions appended so far (the next append's position)."""
        return int(_kv_cache_offset(self._h))

    @property
    def base(self) -> int:
        """Oldest position the cache holds (kv_cache_base)."""
        return int(_kv_cache_base(self._h))

    def append(self, k_rot: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        if k_rot.shape != v.shape or k_rot.dim() != 4:
            raise ValueError("k_rot and v must both be [B, T_new, n_kv, d]")
        if k_rot.dtype != self.dtype or v.dtype != self.dtype:
            raise TypeError("dtype differs from the cache's")
        if (k_rot.shape[0], k_rot.shape[2], k_rot.shape[3]) != (self.B, self.n_kv, self.d):
            raise ValueError("shape differs from the cache's")
        _check(_kv_cache_append(self._h, _dev(k_rot, "k_rot"), _dev(v, "v"),
                                int(k_rot.shape[1]), _stream(stream)))

    def append_rope(self, k: torch.Tensor, v: torch.Tensor, y: "Yarn", stream=None) -> None:
        """kv_cache_append_rope: rotate the unrotated K rows at their cache
        positions (offset + t) and append them with V in one pass."""
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("k and v must both be [B, T_new, n_kv, d]")
        if k.dtype != self.dtype or v.dtype != self.dtype:
            raise TypeError("dtype differs from the cache's")
        if (k.shape[0], k.shape[2], k.shape[3]) != (self.B, self.n_kv, self.d):
            raise ValueError("shape differs from the cache's")
        ys = y.c_struct()
        _check(_kv_cache_append_rope(self._h, _dev(k, "k"), _dev(v, "v"), int(k.shape[1]),
                                     ctypes.byref(ys), _stream(stream)))

    def append_rope_qk(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, y: "Yarn",
                       q_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """kv_cache_append_rope_qk: append_rope that also rotates q [B, T_new,
        n_q, d] at the same positions into q_out (default: a new tensor;
        q_out is q rotates in place); returns q_out."""
        if k.shape != v.shape or k.dim() != 4 or q.dim() != 4:
            raise ValueError("q, k and v must be [B, T_new, heads, d] with k and v alike")
        if q.dtype != self.dtype or k.dtype != self.dtype or v.dtype != self.dtype:
            raise TypeError("dtype differs from the cache's")
        if (k.shape[0], k.shape[2], k.shape[3]) != (self.B, self.n_kv, self.d):
            raise ValueError("shape differs from the cache's")
        if (q.shape[0], q.shape[1], q.shape[3]) != (k.shape[0], k.shape[1], k.shape[3]):
            raise ValueError("q must be [B, T_new, n_q, d] like k")
        if q_out is None:
            q_out = torch.empty_like(q)
        elif q_out.shape != q.shape or q_out.dtype != q.dtype:
            raise ValueError("q_out must match q")
        ys = y.c_struct()
        _check(_kv_cache_append_rope_qk(self._h, _dev(q, "q"), _dev(q_out, "q_out"),
                                        int(q.shape[2]), _dev(k, "k"), _dev(v, "v"),
                                        int(k.shape[1]), ctypes.byref(ys), _stream(stream)))
        return q_out

    def snapshot(self) -> SaSnapshot:
        s = SaSnapshot()
        _check(_kv_cache_snapshot(self._h, ctypes.byref(s)))
        return s

    def restore(self, snap: SaSnapshot) -> None:
        _check(_kv_cache_restore(self._h, ctypes.byref(snap)))

    def v_rows(self) -> torch.Tensor:
        return v_rows(self.v)

    def close(self):
        if getattr(self, "_h", None):
            _kv_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVRing(KVCache):
    """A band layer's ring cache over caller-owned buffers k [B,W,n_kv,d] and
    v [B,W/32,n_kv,d,32]: position p in row p mod W (kv_ring_create).  The
    append methods and sinkattn_decode (window == W) take it directly; a
    prefill chunk goes through a linear stage cache: ``ring.stage(st)``,
    ``st.append_rope_qk(..)``, ``sinkattn_prefill(.., st, .., q_offset=
    ring.offset)``, ``ring.commit(st)``."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor):
        if k.dim() != 4 or v.dim() != 5:
            raise ValueError("k must be [B,W,n_kv,d], v [B,W/32,n_kv,d,32]")
        B, W, n_kv, d = k.shape
        if tuple(v.shape) != v_cache_shape(B, W, n_kv, d) or v.dtype != k.dtype:
            raise ValueError("v buffer shape/dtype does not match k")
        self.k, self.v = k, v
        self.B, self.capacity, self.n_kv, self.d = B, W, n_kv, d
        self.window = W
        self.dtype = k.dtype
        h = _vp()
        _check(_kv_ring_create(ctypes.byref(h), _dev(k, "k"), _dev(v, "v"), _dtype_code(k),
                               B, W, n_kv, d))
        self._h = h

    @classmethod
    def empty(cls, B, W, n_kv, d, dtype=torch.bfloat16, device="cuda", fill=None):
        return super().empty(B, W, n_kv, d, dtype=dtype, device=device, fill=fill)

    def stage(self, stage: KVCache, stream=None) -> KVCache:
        """kv_ring_stage: the stage now holds the ring's rows a query at
        position ``offset`` can see; returns the stage."""
        _check(_kv_ring_stage(stage.handle, self._h, _stream(stream)))
        return stage

    def commit(self, stage: KVCache, stream=None) -> None:
        """kv_ring_commit: the stage's new rows (at most the last W) into the ring."""
        _check(_kv_ring_commit(self._h, stage.handle, _stream(stream)))

    def save(self, k_save: Optional[torch.Tensor] = None, v_save: Optional[torch.Tensor] = None,
             stream=None):
        """kv_ring_save into (new, unless given) buffers shaped like the ring's;
        returns (snapshot, k_save, v_save) for load()."""
        if k_save is None:
            k_save = torch.empty_like(self.k)
        if v_save is None:
            v_save = torch.empty_like(self.v)
        if k_save.shape != self.k.shape or v_save.shape != self.v.shape:
            raise ValueError("save buffers must be shaped like the ring's")
        if k_save.dtype != self.dtype or v_save.dtype != self.dtype:
            raise TypeError("save buffers must have the ring's dtype")
        snap = SaSnapshot()
        _check(_kv_ring_save(self._h, _dev(k_save, "k_save"), _dev(v_save, "v_save"),
                             ctypes.byref(snap), _stream(stream)))
        return snap, k_save, v_save

    def load(self, saved, stream=None) -> None:
        """kv_ring_load of what save() returned."""
        snap, k_save, v_save = saved
        _check(_kv_ring_load(self._h, _dev(k_save, "k_save"), _dev(v_save, "v_save"),
                             ctypes.byref(snap), _stream(stream)))


def sinkattn_prefill(q: torch.Tensor, cache: KVCache, sinks: torch.Tensor, window: int,
                     sm_scale: float, q_offset: int, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """q [B, T_q, n_q, d] (rotated), sinks fp32 [n_q] -> out [B, T_q, n_q, d]."""
    B, T_q, n_q, d = q.shape
    if sinks.dtype != torch.float32 or sinks.numel() != n_q:
        raise ValueError("sinks must be float32 [n_q]")
    if q.dtype != cache.dtype:
        raise TypeError("q dtype differs from the cache's")
    out = _out_like(q, out)
    _check(_sinkattn_prefill(_dev(q, "q"), cache.handle, _dev(sinks, "sinks"), _dev(out, "out"),
                             B, T_q, n_q, cache.n_kv, d, int(window), float(sm_scale),
                             int(q_offset), _stream(stream)))
    return out


def sinkattn_prefill_rope(q: torch.Tensor, cache: KVCache, sinks: torch.Tensor, window: int,
                          sm_scale: float, q_offset: int, y: Yarn,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sinkattn_prefill with unrotated q: each query row is rotated at its
    position q_offset + t inside the kernel (same bits as yarn_rope_apply
    followed by sinkattn_prefill)."""
    B, T_q, n_q, d = q.shape
    if sinks.dtype != torch.float32 or sinks.numel() != n_q:
        raise ValueError("sinks must be float32 [n_q]")
    if q.dtype != cache.dtype:
        raise TypeError("q dtype differs from the cache's")
    out = _out_like(q, out)
    ys = y.c_struct()
    _check(_sinkattn_prefill_rope(_dev(q, "q"), cache.handle, _dev(sinks, "sinks"),
                                  _dev(out, "out"), B, T_q, n_q, cache.n_kv, d, int(window),
                                  float(sm_scale), int(q_offset), ctypes.byref(ys),
                                  _stream(stream)))
    return out


def qkv_workspace_bytes(T: int, d: int) -> int:
    return int(_sinkattn_qkv_ws(int(T), int(d)))


def qkv_rope_append(cache: KVCache, x: torch.Tensor, w_qkv: torch.Tensor, b_qkv: torch.Tensor,
                    n_q: int, y: "Yarn", q_out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sinkattn_qkv_rope_append: x [B, T, d_model] bf16, w_qkv [d_qkv, d_model],
    b_qkv [d_qkv]; writes the rotated queries to q_out [B, T, n_q, d] (new
    if not given) and appends K, V to the cache.  Returns q_out."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, d_model]")
    B, T, dm = x.shape
    d, n_kv = cache.d, cache.n_kv
    dq = d * (n_q + 2 * n_kv)
    if tuple(w_qkv.shape) != (dq, dm) or tuple(b_qkv.shape) != (dq,):
        raise ValueError("w_qkv must be [d (n_q + 2 n_kv), d_model] and b_qkv [d_qkv]")
    if q_out is None:
        q_out = torch.empty((B, T, n_q, d), dtype=x.dtype, device=x.device)
    elif tuple(q_out.shape) != (B, T, n_q, d) or q_out.dtype != x.dtype:
        raise ValueError("q_out must be [B, T, n_q, d] of x's dtype")
    need = qkv_workspace_bytes(T, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    ys = y.c_struct()
    _check(_sinkattn_qkv(cache.handle, _dev(x, "x"), _dev(w_qkv, "w_qkv"), _dev(b_qkv, "b_qkv"),
                         _dev(q_out, "q_out"), B, T, dm, int(n_q), ctypes.byref(ys),
                         _dev(workspace, "workspace"), _nbytes(workspace),
                         _stream(stream)))
    return q_out


def moe_route(x: torch.Tensor, w_router: torch.Tensor, k: int, stream=None):
    """moe_route: x [N, d_model], w_router [E, d_model] (bf16) -> (logits bf16
    [N, E], expert ids int32 [N, k], weights float32 [N, k])."""
    N, dm = x.shape
    E = w_router.shape[0]
    logits = torch.empty((N, E), dtype=torch.bfloat16, device=x.device)
    ids = torch.empty((N, k), dtype=torch.int32, device=x.device)
    w = torch.empty((N, k), dtype=torch.float32, device=x.device)
    _check(_moe_route(_dev(x, "x"), N, dm, _dev(w_router, "w_router"), E, int(k),
                      _dev(logits, "logits"), _dev(ids, "ids"), _dev(w, "weights"), _stream(stream)))
    return logits, ids, w


def moe_dispatch(ids: torch.Tensor, E: int, stream=None):
    """moe_dispatch: ids int32 [N, k] -> (rows int32 [N*k] = token*k + slot
    grouped by expert then token, expert_start int32 [E+1])."""
    N, k = ids.shape
    rows = torch.empty(N * k, dtype=torch.int32, device=ids.device)
    start = torch.empty(E + 1, dtype=torch.int32, device=ids.device)
    ws = torch.empty(max(int(_moe_dispatch_ws(N, E)), 16), dtype=torch.uint8, device=ids.device)
    _check(_moe_dispatch(_dev(ids, "ids"), N, int(E), k, _dev(rows, "rows"), _dev(start, "start"),
                         _dev(ws, "workspace"), _nbytes(ws), _stream(stream)))
    return rows, start


def moe_workspace_bytes(N, d_model, E, k, ffn, ffn_shared=0) -> int:
    return int(_moe_ws(N, d_model, E, k, ffn, ffn_shared))


def moe_layer(x: torch.Tensor, w_router: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, k: int,
              shared=None, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_layer: x [N, d_model]; w_router [E, d_model]; w13 [E, 2 ffn,
    d_model]; w2 [E, d_model, ffn]; shared = (w13s [2 ffn_s, d_model], w2s
    [d_model, ffn_s]) or None.  Returns y [N, d_model] bf16."""
    N, dm = x.shape
    E, two_ffn, _ = w13.shape
    ffn = two_ffn // 2
    if shared is not None:
        w13s, w2s = shared
        ffn_s = w13s.shape[0] // 2
        p13, p2 = _dev(w13s, "w13_shared"), _dev(w2s, "w2_shared")
    else:
        ffn_s, p13, p2 = 0, None, None
    if out is None:
        out = torch.empty((N, dm), dtype=torch.bfloat16, device=x.device)
    need = moe_workspace_bytes(N, dm, E, k, ffn, ffn_s)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(_moe_layer(_dev(x, "x"), N, dm, _dev(w_router, "w_router"), E, int(k), _dev(w13, "w13"),
                      _dev(w2, "w2"), ffn, p13, p2, ffn_s, _dev(out, "out"),
                      _dev(workspace, "workspace"), _nbytes(workspace),
                      _stream(stream)))
    return out


def decode_workspace_bytes(B, n_q, n_kv, d, capacity) -> int:
    return int(_sinkattn_decode_ws(B, n_q, n_kv, d, capacity))


def decode_workspace(cache: KVCache, n_q: int) -> torch.Tensor:
    n = decode_workspace_bytes(cache.B, n_q, cache.n_kv, cache.d, cache.capacity)
    return torch.empty(max(1, n // 4), dtype=torch.float32, device=cache.k.device)


def sinkattn_decode(q: torch.Tensor, cache: KVCache, sinks: torch.Tensor, window: int,
                    sm_scale: float, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [B, 1, n_q, d] of the token at position cache.offset - 1."""
    B, T1, n_q, d = q.shape
    if T1 != 1:
        raise ValueError("decode takes exactly one query token per sequence")
    if sinks.dtype != torch.float32 or sinks.numel() != n_q:
        raise ValueError("sinks must be float32 [n_q]")
    if q.dtype != cache.dtype:
        raise TypeError("q dtype differs from the cache's")
    if workspace is None:
        workspace = decode_workspace(cache, n_q)
    out = _out_like(q, out)
    _check(_sinkattn_decode(_dev(q, "q"), cache.handle, _dev(sinks, "sinks"), _dev(out, "out"),
                            B, n_q, cache.n_kv, d, int(window), float(sm_scale),
                            _dev(workspace, "workspace"), _nbytes(workspace),
                            _stream(stream)))
    return out


def sinkattn_decode_noalloc(q: torch.Tensor, cache: KVCache, sinks: torch.Tensor, window: int,
                            sm_scale: float, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """sinkattn_decode without a workspace: the split partials live in the
    library's static per-GPU scratch (calls on one GPU must not overlap)."""
    B, T1, n_q, d = q.shape
    if T1 != 1:
        raise ValueError("decode takes exactly one query token per sequence")
    if sinks.dtype != torch.float32 or sinks.numel() != n_q:
        raise ValueError("sinks must be float32 [n_q]")
    if q.dtype != cache.dtype:
        raise TypeError("q dtype differs from the cache's")
    out = _out_like(q, out)
    _check(_sinkattn_decode_noalloc(_dev(q, "q"), cache.handle, _dev(sinks, "sinks"),
                                    _dev(out, "out"), B, n_q, cache.n_kv, d, int(window),
                                    float(sm_scale), _stream(stream)))
    return out


def sinkattn_decode_step(cache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         sinks: torch.Tensor, window: int, sm_scale: float, y: "Yarn",
                         q_rot: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One fused decode step: q [B, 1, n_q, d] and k, v [B, 1, n_kv, d] of the
    token at position cache.offset, unrotated; rotates them, appends the K/V
    row and attends (bf16).  q_rot, if given, receives the rotated q."""
    B, T1, n_q, d = q.shape
    if T1 != 1 or k.shape != (B, 1, cache.n_kv, d) or v.shape != k.shape:
        raise ValueError("q must be [B, 1, n_q, d] and k, v [B, 1, n_kv, d]")
    if sinks.dtype != torch.float32 or sinks.numel() != n_q:
        raise ValueError("sinks must be float32 [n_q]")
    if q.dtype != cache.dtype or k.dtype != cache.dtype or v.dtype != cache.dtype:
        raise TypeError("dtype differs from the cache's")
    if workspace is None:
        workspace = decode_workspace(cache, n_q)
    out = _out_like(q, out)
    qr = 0
    if q_rot is not None:
        if q_rot.shape != q.shape or q_rot.dtype != q.dtype:
            raise ValueError("q_rot must match q")
        qr = _dev(q_rot, "q_rot")
    ys = y.c_struct()
    _check(_sinkattn_decode_step(cache.handle, _dev(q, "q"), qr, _dev(k, "k"), _dev(v, "v"),
                                 _dev(sinks, "sinks"), _dev(out, "out"), B, n_q, cache.n_kv, d,
                                 int(window), float(sm_scale), ctypes.byref(ys),
                                 _dev(workspace, "workspace"), _nbytes(workspace),
                                 _stream(stream)))
    return out


def decode_scratch_bytes() -> int:
    return int(_sinkattn_decode_scratch_bytes())


def sample_params(B: int, temperature=1.0, top_k=0, top_p=1.0, min_p=0.0, repetition=1.0,
                  presence=0.0, frequency=0.0, device="cuda") -> torch.Tensor:
    """Per-row sampling parameters (each a scalar or a sequence of B values)
    packed as B sa_sample_params structs in a device uint8 tensor."""
    arr = (SaSampleParams * B)()
    cols = dict(temperature=temperature, top_k=top_k, top_p=top_p, min_p=min_p,
                repetition=repetition, presence=presence, frequency=frequency)
    for name, val in cols.items():
        vals = list(val) if hasattr(val, "__len__") else [val] * B
        if len(vals) != B:
            raise ValueError("%s: %d values for %d rows" % (name, len(vals), B))
        for i, x in enumerate(vals):
            setattr(arr[i], name, int(x) if name == "top_k" else float(x))
    raw = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return raw.to(device)


def sample_workspace_bytes(B: int, V: int) -> int:
    return int(_sample_ws(B, V))


def sample_count_tokens(ids: torch.Tensor, counts: torch.Tensor, stream=None) -> torch.Tensor:
    """counts[b, id] += 1 for every id of ids [B, H] (int32) in [0, V);
    counts: int32 [B, V], updated in place."""
    B, H = ids.shape
    V = counts.shape[1]
    _check(_sample_count_tokens(_dev(ids, "ids") if H else None, B, H, H, _dev(counts, "counts"), V,
                                _stream(stream)))
    return counts


def sample_tokens(logits: torch.Tensor, params: torch.Tensor, u: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None,
                  update_counts: bool = False, want_kept: bool = False, want_processed: bool = False,
                  workspace: Optional[torch.Tensor] = None, stream=None):
    """sample_tokens: logits fp32 [B, V]; params from sample_params; u fp32 [B];
    bias fp32 [V] (shared) or [B, V], or None; counts int32 [B, V] or None.
    Returns tokens int32 [B], plus n_kept int32 [B] and / or the processed
    logits fp32 [B, V] when asked for."""
    B, V = logits.shape
    if bias is not None:
        bias_stride = 0 if bias.dim() == 1 else bias.shape[1]
        pb = _dev(bias, "bias")
    else:
        bias_stride, pb = 0, None
    tokens = torch.empty(B, dtype=torch.int32, device=logits.device)
    kept = torch.empty(B, dtype=torch.int32, device=logits.device) if want_kept else None
    proc = torch.empty((B, V), dtype=torch.float32, device=logits.device) if want_processed else None
    need = sample_workspace_bytes(B, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    _check(_sample_tokens(_dev(logits, "logits"), B, V, V, pb, bias_stride,
                          _dev(counts, "counts") if counts is not None else None,
                          _dev(params, "params"), _dev(u, "u"), 1 if update_counts else 0,
                          _dev(tokens, "tokens"), _dev(kept, "n_kept") if kept is not None else None,
                          _dev(proc, "processed") if proc is not None else None,
                          _dev(workspace, "workspace"), _nbytes(workspace),
                          _stream(stream)))
    out = [tokens]
    if want_kept:
        out.append(kept)
    if want_processed:
        out.append(proc)
    return tokens if len(out) == 1 else tuple(out)
