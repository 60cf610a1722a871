"""CPU oracle for the attention hot path: plain fp64 C behind a thin numpy/ctypes shim.

TEST INFRASTRUCTURE ONLY -- the test-suite, the smoke check and the benchmark's CPU
baseline are its only callers.  It shares no code with the GPU library.

Every tensor crosses this shim as raw IEEE binary16 bits in ``numpy.uint16`` arrays
(positions and lengths as ``int32``), with the layouts

    q, out      [n, t, hq, d]        k, v (new)   [n, t, hkv, d]
    positions   [n, t]               lens         [n]
    cache_k/v   [n, hkv, s_cap, d]   (updated in place)

The arithmetic lives in ``kvrope_oracle.c``; see its header for the passages of the pages
each function follows.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import math
import os

import numpy as np

from . import build as _build

_lib = None


@dataclasses.dataclass(frozen=True, eq=False)
class RopeParams:
    base: float = 10000.0
    n_rot: int = 128
    yarn: bool = False
    freq_scale: float = 1.0
    ext_factor: float = 0.0
    n_ctx_orig: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    half_split: bool = False       # pairs (o + j, o + j + n_rot/2) instead of (o + 2j, o + 2j + 1)
    inverse: bool = False          # rotate by -theta
    cos_table: np.ndarray | None = None  # float32 [rows, n_rot/2], gathered by position
    sin_table: np.ndarray | None = None

    def replace(self, **kw) -> "RopeParams":
        return dataclasses.replace(self, **kw)

    @staticmethod
    def plain(n_rot: int = 128, base: float = 10000.0) -> "RopeParams":
        return RopeParams(base=base, n_rot=n_rot)

    @staticmethod
    def yarn_tail(n_rot: int = 64, base: float = 10000.0, factor: float = 4.0,
                  n_ctx_orig: int = 4096, beta_fast: float = 32.0,
                  beta_slow: float = 1.0) -> "RopeParams":
        return RopeParams(base=base, n_rot=n_rot, yarn=True, freq_scale=1.0 / factor,
                          ext_factor=1.0, n_ctx_orig=n_ctx_orig, beta_fast=beta_fast,
                          beta_slow=beta_slow, mscale=1.0 + 0.1 * math.log(factor))


class _CRope(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("n_rot", ctypes.c_int32), ("yarn", ctypes.c_int32),
                ("freq_scale", ctypes.c_double), ("ext_factor", ctypes.c_double),
                ("n_ctx_orig", ctypes.c_int32), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("mscale", ctypes.c_double),
                ("pairing", ctypes.c_int32), ("inverse", ctypes.c_int32),
                ("cos_table", ctypes.c_void_p), ("sin_table", ctypes.c_void_p),
                ("table_rows", ctypes.c_int32)]


def _table(a, half: int) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    assert a.ndim == 2 and a.shape[1] == half, a.shape
    return a


def _c_rope(rp: RopeParams) -> _CRope:
    """The C parameter block.  It points into rp's tables: keep rp alive while it is used."""
    c = _CRope(rp.base, rp.n_rot, int(rp.yarn), rp.freq_scale, rp.ext_factor,
               rp.n_ctx_orig, rp.beta_fast, rp.beta_slow, rp.mscale, int(rp.half_split),
               int(rp.inverse), None, None, 0)
    if (rp.cos_table is None) != (rp.sin_table is None):
        raise ValueError("cos_table and sin_table go together")
    if rp.cos_table is not None:
        ct, st = _table(rp.cos_table, rp.n_rot // 2), _table(rp.sin_table, rp.n_rot // 2)
        assert ct.shape == st.shape
        c.cos_table, c.sin_table, c.table_rows = ct.ctypes.data, st.ctypes.data, ct.shape[0]
        c._keep = (ct, st)
    return c


def _c_rope_sets(rp, unit_set, n: int):
    """(C array of parameter blocks, keep-alive list, unit_set int32 array or None).

    rp is one RopeParams (every unit) or a sequence of them with unit_set [n] naming the
    set each unit uses."""
    sets = [rp] if isinstance(rp, RopeParams) else list(rp)
    if not sets:
        raise ValueError("at least one rotary parameter set is needed")
    arr = (_CRope * len(sets))()
    keep = []
    for i, s in enumerate(sets):
        c = _c_rope(s)
        keep.append(c)
        arr[i] = c
    if unit_set is None:
        if len(sets) != 1:
            raise ValueError("several parameter sets need unit_set")
        return arr, keep, None
    us = np.ascontiguousarray(np.asarray(unit_set, dtype=np.int32))
    if us.shape != (n,) or us.min(initial=0) < 0 or us.max(initial=0) >= len(sets):
        raise ValueError("unit_set must be [n] indices into the parameter sets")
    return arr, keep, us


_P = ctypes.c_void_p


def load(path: str) -> ctypes.CDLL:
    """Load an oracle library build and declare its C signatures."""
    L = ctypes.CDLL(path)
    L.ora_f16_to_f64.restype = ctypes.c_double
    L.ora_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.ora_f64_to_f16.restype = ctypes.c_uint16
    L.ora_f64_to_f16.argtypes = [ctypes.c_double]
    L.ora_f16_to_f64_array.argtypes = [_P, _P, ctypes.c_int64]
    L.ora_f64_to_f16_array.argtypes = [_P, _P, ctypes.c_int64]
    L.ora_yarn_corr_dim.restype = ctypes.c_double
    L.ora_yarn_corr_dim.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_double]
    L.ora_yarn_ramp.restype = ctypes.c_double
    L.ora_yarn_ramp.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int]
    L.ora_rope_freqs.argtypes = [ctypes.POINTER(_CRope), _P, _P, _P]
    L.ora_rope.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                           ctypes.POINTER(_CRope), _P, _P]
    L.ora_append.restype = ctypes.c_int
    L.ora_append.argtypes = [_P, _P, _P, _P, _P] + [ctypes.c_int] * 5
    L.ora_prefill_kv.restype = ctypes.c_int
    L.ora_prefill_kv.argtypes = ([_P] * 8 + [ctypes.c_int] * 6 +
                                 [ctypes.c_double, _P, _P, _P, _P])
    L.ora_decode.restype = ctypes.c_int
    L.ora_decode.argtypes = ([_P] * 8 + [ctypes.c_int] * 5 +
                             [ctypes.c_double, _P, _P, _P, _P])
    L.ora_num_threads.restype = ctypes.c_int
    L.ora_set_num_threads.argtypes = [ctypes.c_int]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load(_build.LIB)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another build (mutation tests)."""
    global _lib
    prev = lib()
    _lib = load(path)
    try:
        yield
    finally:
        _lib = prev


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads() -> int:
    return lib().ora_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use (for timing runs; results do not depend on it)."""
    lib().ora_set_num_threads(int(n))


# ---------------------------------------------------------------- f16 codec
def f16_to_f64(h) -> np.ndarray:
    h = _u16(h)
    out = np.empty(h.shape, dtype=np.float64)
    lib().ora_f16_to_f64_array(_ptr(h), _ptr(out), h.size)
    return out


def f64_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().ora_f64_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


# ---------------------------------------------------------------- RoPE
def yarn_corr_dim(n_dims: int, n_ctx_orig: int, beta: float, base: float) -> float:
    return lib().ora_yarn_corr_dim(n_dims, n_ctx_orig, beta, base)


def yarn_ramp(low: float, high: float, j: int) -> float:
    return lib().ora_yarn_ramp(low, high, j)


def rope_freqs(rp: RopeParams):
    """Returns (omega_eff[n_rot/2], gamma[n_rot/2], (d0, d1))."""
    half = rp.n_rot // 2
    om = np.empty(max(half, 1), dtype=np.float64)
    ga = np.empty(max(half, 1), dtype=np.float64)
    dims = np.empty(2, dtype=np.float64)
    c = _c_rope(rp)
    lib().ora_rope_freqs(ctypes.byref(c), _ptr(om), _ptr(ga), _ptr(dims))
    return om[:half], ga[:half], (float(dims[0]), float(dims[1]))


def rope(x, positions, rp: RopeParams):
    """x: [rows, h, d] f16 bits, positions: [rows].  Returns (rotated f16 bits, fp64)."""
    x = _u16(x)
    pos = _i32(positions)
    rows, h, d = x.shape
    assert pos.shape == (rows,)
    out = np.empty_like(x)
    out64 = np.empty(x.shape, dtype=np.float64)
    c = _c_rope(rp)
    lib().ora_rope(_ptr(x), _ptr(pos), rows, h, d, ctypes.byref(c), _ptr(out), _ptr(out64))
    return out, out64


# ---------------------------------------------------------------- projections
def project(a, w) -> tuple:
    """y = a . w^T ([Sophgo] Listings 1-2: MatMul(x, w) with w stored one row per output
    feature).  a [..., K], w [N, K] f16 bits.  Every product of two f16 values is exact in
    fp64 and the sum of K of them keeps ~53 bits, so the result is the exact dot product to
    within far less than an f16 ulp.  Returns (fp64 [..., N], RNE f16 bits)."""
    a64 = f16_to_f64(a)
    w64 = f16_to_f64(w)
    y = a64 @ w64.T
    return y, f64_to_f16(y)


def qkv_project(x, w_qkv, hq: int, hkv: int, d: int = 128):
    """x [n, t, hidden], w_qkv [(hq + 2 hkv) d, hidden] (or one per unit: [n, ...]) f16 bits.
    Returns the f16 q [n,t,hq,d], k [n,t,hkv,d], v [n,t,hkv,d] of the projection."""
    x, w = _u16(x), _u16(w_qkv)
    n, t, _ = x.shape
    if w.ndim == 2:
        _, y = project(x.reshape(n * t, -1), w)
        y = y.reshape(n, t, -1)
    else:
        y = np.stack([project(x[u], w[u])[1] for u in range(n)])
    q = y[..., : hq * d].reshape(n, t, hq, d)
    k = y[..., hq * d: (hq + hkv) * d].reshape(n, t, hkv, d)
    v = y[..., (hq + hkv) * d:].reshape(n, t, hkv, d)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def out_project(attn, w_o, residual):
    """out = attn . w_o^T + residual ([Sophgo] Listings 1-2: Add(input, MatMul(attn, w_o))),
    rounded once to f16.  attn [n, t, F], w_o [hidden, F] (or [n, hidden, F]), residual
    [n, t, hidden] f16 bits.  Returns (fp64, f16 bits)."""
    attn, w, res = _u16(attn), _u16(w_o), _u16(residual)
    n, t = attn.shape[:2]
    a = attn.reshape(n, t, -1)
    if w.ndim == 2:
        y = project(a.reshape(n * t, -1), w)[0].reshape(n, t, -1)
    else:
        y = np.stack([project(a[u], w[u])[0] for u in range(n)])
    y = y + f16_to_f64(res)
    return y, f64_to_f16(y)


# ---------------------------------------------------------------- cache append
def append(cache_k: np.ndarray, cache_v: np.ndarray, k, v, lens) -> None:
    """In place: rows [lens[n], lens[n]+t) of each cache get k / v (bit copy)."""
    k, v, lens = _u16(k), _u16(v), _i32(lens)
    n, t, hkv, d = k.shape
    s_cap = cache_k.shape[2]
    assert cache_k.shape == (n, hkv, s_cap, d) and cache_v.shape == cache_k.shape
    rc = lib().ora_append(_ptr(cache_k), _ptr(cache_v), _ptr(k), _ptr(v), _ptr(lens),
                          n, t, hkv, d, s_cap)
    if rc != 0:
        raise ValueError("oracle append: capacity exceeded")


# ---------------------------------------------------------------- attention
def prefill_kv(q, k, v, positions, cache_k: np.ndarray, cache_v: np.ndarray, lens,
               scale: float, rp, unit_set=None):
    """Chunked prefill over a history.  Caches are updated in place.  rp: one RopeParams,
    or a list of them with unit_set [n] choosing each unit's set.

    Returns (out f16 bits [n,t,hq,d], out fp64, rotated k fp64 [n,t,hkv,d])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    pos, lens = _i32(positions), _i32(lens)
    n, t, hq, d = q.shape
    hkv = k.shape[2]
    s_cap = cache_k.shape[2]
    assert k.shape == (n, t, hkv, d) and v.shape == k.shape and pos.shape == (n, t)
    assert cache_k.shape == (n, hkv, s_cap, d) and cache_v.shape == cache_k.shape
    assert cache_k.dtype == np.uint16 and cache_k.flags["C_CONTIGUOUS"]
    assert cache_v.dtype == np.uint16 and cache_v.flags["C_CONTIGUOUS"]
    assert lens.shape == (n,)
    out = np.empty(q.shape, dtype=np.uint16)
    out64 = np.empty(q.shape, dtype=np.float64)
    k64 = np.empty(k.shape, dtype=np.float64)
    sets, _keep, us = _c_rope_sets(rp, unit_set, n)
    rc = lib().ora_prefill_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(cache_k),
                              _ptr(cache_v), _ptr(lens), _ptr(out), n, t, hq, hkv, d, s_cap,
                              float(scale), ctypes.cast(sets, ctypes.c_void_p),
                              None if us is None else _ptr(us), _ptr(out64), _ptr(k64))
    if rc != 0:
        raise ValueError("oracle prefill_kv: shape or capacity error")
    return out, out64, k64


def prefill_kv_varlen(q, k, v, positions, cache_k: np.ndarray, cache_v: np.ndarray, lens, new_lens,
                      scale: float, rp, unit_set=None):
    """prefill_kv over a batch whose unit u brings new_lens[u] new tokens (rows past it are
    padding): unit u is prefill_kv of that unit alone on its first new_lens[u] rows ([Sophgo]
    Listing 2 per sequence).  Caches are updated in place.  Returns (out bits, out fp64,
    rotated k fp64) with NaN / 0 bits in the padding rows."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    pos, lens, nl = _i32(positions), _i32(lens), _i32(new_lens)
    n, t = q.shape[:2]
    out = np.zeros(q.shape, dtype=np.uint16)
    out64 = np.full(q.shape, np.nan)
    k64 = np.full(k.shape, np.nan)
    for u in range(n):
        tu = int(nl[u])
        if not 0 <= tu <= t:
            raise ValueError("oracle prefill_kv_varlen: new_lens out of range")
        if tu == 0:
            continue
        ck, cv = np.ascontiguousarray(cache_k[u:u + 1]), np.ascontiguousarray(cache_v[u:u + 1])
        rpu = rp if unit_set is None else list(rp)[int(unit_set[u])]
        o, o64, kk = prefill_kv(q[u:u + 1, :tu], k[u:u + 1, :tu], v[u:u + 1, :tu], pos[u:u + 1, :tu],
                                ck, cv, lens[u:u + 1], scale, rpu)
        cache_k[u], cache_v[u] = ck[0], cv[0]
        out[u, :tu], out64[u, :tu], k64[u, :tu] = o[0], o64[0], kk[0]
    return out, out64, k64


def prefill(q, k, v, positions, cache_k, cache_v, scale: float, rp, unit_set=None):
    n = np.asarray(q).shape[0]
    return prefill_kv(q, k, v, positions, cache_k, cache_v, np.zeros(n, np.int32), scale, rp,
                      unit_set)


def decode(q, k, v, positions, cache_k: np.ndarray, cache_v: np.ndarray, lens, scale: float,
           rp, unit_set=None):
    """One decode step.  q: [n, hq, d]; k, v: [n, hkv, d]; positions, lens: [n].  rp and
    unit_set as for prefill_kv.

    Caches are updated in place (row lens[n]).  Returns (out bits [n,hq,d], out fp64,
    rotated k fp64 [n,hkv,d])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    pos, lens = _i32(positions), _i32(lens)
    n, hq, d = q.shape
    hkv = k.shape[1]
    s_cap = cache_k.shape[2]
    assert k.shape == (n, hkv, d) and v.shape == k.shape and pos.shape == (n,)
    assert cache_k.shape == (n, hkv, s_cap, d) and cache_v.shape == cache_k.shape
    assert cache_k.dtype == np.uint16 and cache_k.flags["C_CONTIGUOUS"]
    out = np.empty(q.shape, dtype=np.uint16)
    out64 = np.empty(q.shape, dtype=np.float64)
    k64 = np.empty(k.shape, dtype=np.float64)
    sets, _keep, us = _c_rope_sets(rp, unit_set, n)
    rc = lib().ora_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(cache_k), _ptr(cache_v),
                          _ptr(lens), _ptr(out), n, hq, hkv, d, s_cap, float(scale),
                          ctypes.cast(sets, ctypes.c_void_p), None if us is None else _ptr(us),
                          _ptr(out64), _ptr(k64))
    if rc != 0:
        raise ValueError("oracle decode: shape or capacity error")
    return out, out64, k64

