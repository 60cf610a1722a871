"""kv_cache_causal_rope_amd -- Python binding of libkvrope, the MI355X (gfx950) attention
hot path: rotary embedding of Q/K (plain or YaRN tail rotation), KV-cache append and
causal grouped-query attention in the prefill / prefill_kv / decode phases.

This module only marshals arguments: it checks dtypes, devices and shapes of torch
tensors and hands raw device pointers and the current HIP stream to the C ABI declared in
``include/kvrope.h``.  Every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if ``libkvrope.so`` is missing the calls raise.

Layouts (f16, contiguous, innermost last):
    q, out [n, t, hq, 128]   k, v [n, t, hkv, 128]   caches [n, hkv, s_cap, 128]
    positions int32 [n, t]   lens int32 [n]
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch  # imported first: the library binds to the HIP runtime torch has loaded

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvrope.so")

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_ROPE = -3
ATTN_ERR_CAPACITY = -4
ATTN_ERR_ALIGN = -5
ATTN_ERR_WORKSPACE = -6
ATTN_ERR_SCALE = -7
ATTN_ERR_HIP = -8
ATTN_OP_DECODE = 1
MAX_ROPE_SETS = 4

# every symbol include/kvrope.h declares
EXPORTS = ["attn_rope_apply", "kv_cache_append", "attn_prefill", "attn_prefill_kv",
           "attn_prefill_kv_varlen", "attn_decode", "attn_workspace_size", "attn_status_string",
           "attn_last_hip_error", "attn_set_profile_events", "attn_qkv_project", "attn_out_project",
           "attn_prefill_kv_cached", "attn_decode_noalloc", "attn_decode_noalloc_max_workspace",
           "attn_decode_chunk_keys"]


class KVRopeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvrope status {status}: {message}")
        self.status = status


class RopeParams(ctypes.Structure):
    """Mirror of ``kvrope_rope_params``.

    ``with_variant`` sets the half-split pairing, the inverse rotation and the caller's
    cos / sin tables (CUDA float32 tensors [rows, n_rot / 2]; the struct keeps them alive).
    ``with_sets`` gives each unit its own frequency parameters.
    """


RopeParams._fields_ = [("base", ctypes.c_double), ("n_rot", ctypes.c_int32), ("yarn", ctypes.c_int32),
                       ("freq_scale", ctypes.c_double), ("ext_factor", ctypes.c_double),
                       ("n_ctx_orig", ctypes.c_int32), ("beta_fast", ctypes.c_double),
                       ("beta_slow", ctypes.c_double), ("mscale", ctypes.c_double),
                       ("pairing", ctypes.c_int32), ("inverse", ctypes.c_int32),
                       ("cos_table", ctypes.c_void_p), ("sin_table", ctypes.c_void_p),
                       ("table_rows", ctypes.c_int32), ("n_sets", ctypes.c_int32),
                       ("sets", ctypes.POINTER(RopeParams)), ("unit_set", ctypes.c_void_p)]


def _plain(cls, n_rot: int = 128, base: float = 10000.0) -> "RopeParams":
    return cls(base, n_rot, 0, 1.0, 0.0, 4096, 32.0, 1.0, 1.0)


def _with_variant(self, half_split: bool = False, inverse: bool = False, cos_table=None,
                  sin_table=None) -> "RopeParams":
    """A copy with the given pairing, direction and tables."""
    r = RopeParams.from_buffer_copy(self)
    r.pairing, r.inverse = int(half_split), int(inverse)
    if (cos_table is None) != (sin_table is None):
        raise ValueError("cos_table and sin_table go together")
    if cos_table is not None:
        for tt in (cos_table, sin_table):
            if not (tt.is_cuda and tt.dtype == torch.float32 and tt.is_contiguous() and tt.dim() == 2
                    and tt.shape == cos_table.shape and tt.shape[1] == self.n_rot // 2):
                raise ValueError("tables must be contiguous CUDA float32 [rows, n_rot / 2]")
        r.cos_table, r.sin_table = cos_table.data_ptr(), sin_table.data_ptr()
        r.table_rows = cos_table.shape[0]
        r._keep = (cos_table, sin_table)
    else:
        r.cos_table = r.sin_table = None
        r.table_rows = 0
    r.n_sets, r.sets, r.unit_set = 0, None, None
    return r


def _with_sets(self, sets, unit_set: torch.Tensor) -> "RopeParams":
    """A copy whose unit u takes its frequency fields (base, YaRN fields, mscale) from
    sets[unit_set[u]] (1 <= len(sets) <= MAX_ROPE_SETS; unit_set a CUDA int32 [n] tensor);
    n_rot, pairing and inverse stay this struct's."""
    sets = list(sets)
    if not (isinstance(unit_set, torch.Tensor) and unit_set.is_cuda and unit_set.dtype == torch.int32
            and unit_set.is_contiguous() and unit_set.dim() == 1):
        raise ValueError("unit_set must be a contiguous CUDA int32 [n] tensor")
    arr = (RopeParams * len(sets))(*[RopeParams.from_buffer_copy(x) for x in sets])
    r = RopeParams.from_buffer_copy(self)
    r.n_sets = len(sets)
    r.sets = ctypes.cast(arr, ctypes.POINTER(RopeParams))
    r.unit_set = unit_set.data_ptr()
    r._keep = (arr, unit_set, getattr(self, "_keep", None))
    return r


def _yarn_tail(cls, n_rot: int = 64, base: float = 10000.0, factor: float = 4.0,
               n_ctx_orig: int = 4096, beta_fast: float = 32.0, beta_slow: float = 1.0,
               mscale: Optional[float] = None) -> "RopeParams":
    if mscale is None:
        mscale = 1.0 + 0.1 * math.log(factor)
    return cls(base, n_rot, 1, 1.0 / factor, 1.0, n_ctx_orig, beta_fast, beta_slow, mscale)


def _from_fields(cls, r) -> "RopeParams":
    """From any object with the same field names (e.g. a workload's Rope)."""
    return cls(r.base, r.n_rot, int(r.yarn), r.freq_scale, r.ext_factor, r.n_ctx_orig,
               r.beta_fast, r.beta_slow, r.mscale)


RopeParams.plain = classmethod(_plain)
RopeParams.with_variant = _with_variant
RopeParams.with_sets = _with_sets
RopeParams.yarn_tail = classmethod(_yarn_tail)
RopeParams.from_fields = classmethod(_from_fields)


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def _count_hip_runtimes() -> int:
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
        return len(paths)
    except OSError:
        return 1


def lib() -> ctypes.CDLL:
    """Load libkvrope.so (built by ``python -m kv_cache_causal_rope_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m kv_cache_causal_rope_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    if _count_hip_runtimes() > 1:
        raise RuntimeError("more than one libamdhip64 is mapped into this process; "
                           "libkvrope must share torch's HIP runtime")
    rp = ctypes.POINTER(RopeParams)
    L.attn_rope_apply.argtypes = [_P, _P, _I, _I, _I, _I, rp, _P]
    L.kv_cache_append.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
    L.attn_prefill.argtypes = [_P] * 7 + [_I] * 6 + [ctypes.c_double, rp, _P]
    L.attn_prefill_kv.argtypes = ([_P] * 7 + [_I, _P] + [_I] * 6 +
                                  [ctypes.c_double, rp, _P])
    L.attn_prefill_kv_varlen.argtypes = ([_P] * 7 + [_I, _P, _P] + [_I] * 6 +
                                         [ctypes.c_double, rp, _P])
    L.attn_decode.argtypes = ([_P] * 7 + [_I, _P] + [_I] * 5 +
                              [ctypes.c_double, rp, _P, ctypes.c_size_t, _P])
    L.attn_decode_noalloc.argtypes = ([_P] * 7 + [_I, _P] + [_I] * 5 + [ctypes.c_double, rp, _P])
    L.attn_decode_noalloc_max_workspace.argtypes = []
    L.attn_decode_noalloc_max_workspace.restype = ctypes.c_size_t
    L.attn_decode_chunk_keys.argtypes = [_I] * 4
    L.attn_decode_chunk_keys.restype = _I
    L.attn_workspace_size.argtypes = [_I] * 7
    L.attn_workspace_size.restype = ctypes.c_size_t
    L.attn_status_string.argtypes = [_I]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_hip_error.restype = _I
    L.attn_set_profile_events.argtypes = [_P, _P]
    L.attn_qkv_project.argtypes = [_P, _P, _I, _P, _P, _P, _P, _P] + [_I] * 8 + [rp, _P]
    L.attn_out_project.argtypes = [_P, _P, _I, _P, _P] + [_I] * 5 + [_P]
    L.attn_prefill_kv_cached.argtypes = [_P] * 5 + [_I, _P] + [_I] * 6 + [ctypes.c_double, rp, _P]
    for rtn in ["attn_rope_apply", "kv_cache_append", "attn_prefill", "attn_prefill_kv",
                "attn_prefill_kv_varlen", "attn_decode", "attn_set_profile_events", "attn_qkv_project",
                "attn_out_project", "attn_prefill_kv_cached", "attn_decode_noalloc"]:
        getattr(L, rtn).restype = _I
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


def _check(status: int) -> None:
    if status != ATTN_OK:
        msg = status_string(status)
        if status == ATTN_ERR_HIP:
            msg += f" (hipError {lib().attn_last_hip_error()})"
        raise KVRopeError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _f16(name: str, t: torch.Tensor, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda:
        raise TypeError(f"{name} must be a float16 CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _i32(name: str, t: torch.Tensor, shape) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda:
        raise TypeError(f"{name} must be an int32 CUDA tensor")
    if not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}")
    return t


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc(stream, make):
    """Allocate with `make()` in the caching allocator's pool of the stream the kernels run
    on, so that torch does not hand the memory to other work while those kernels may still
    use it."""
    if stream is None:
        return make()
    with torch.cuda.stream(stream):
        return make()


def decode_chunk_keys(n: int, hq: int, hkv: int, max_len: int) -> int:
    """Keys per chunk (at most) attn_decode splits a unit's keys into for this shape."""
    return int(lib().attn_decode_chunk_keys(n, hq, hkv, max_len))


def workspace_size(n: int, hq: int, hkv: int, max_len: int, d: int = 128) -> int:
    return int(lib().attn_workspace_size(ATTN_OP_DECODE, n, 1, hq, hkv, d, max_len))


def set_profile_events(before: Optional[torch.cuda.Event], after: Optional[torch.cuda.Event]):
    """Record `before` / `after` around the attention kernel of the calling thread's next
    prefill / decode call (events must have been created on the current device)."""
    b = ctypes.c_void_p(before.cuda_event) if before is not None else None
    a = ctypes.c_void_p(after.cuda_event) if after is not None else None
    _check(lib().attn_set_profile_events(b, a))


def rope_apply(x: torch.Tensor, positions: torch.Tensor, rope: RopeParams, stream=None):
    """Rotate x [n, t, h, 128] in place at positions [n, t]."""
    n, t, h, d = x.shape
    _f16("x", x)
    _i32("positions", positions, (n, t))
    _check(lib().attn_rope_apply(_ptr(x), _ptr(positions), n, t, h, d, ctypes.byref(rope),
                                 _stream(stream)))
    return x


def cache_append(cache_k, cache_v, k, v, lens, max_len: int, stream=None):
    """Copy k, v [n, t, hkv, 128] to cache rows [lens[u], lens[u] + t)."""
    n, t, hkv, d = k.shape
    s_cap = cache_k.shape[2]
    _f16("cache_k", cache_k, (n, hkv, s_cap, d))
    _f16("cache_v", cache_v, (n, hkv, s_cap, d))
    _f16("k", k)
    _f16("v", v, k.shape)
    _i32("lens", lens, (n,))
    _check(lib().kv_cache_append(_ptr(cache_k), _ptr(cache_v), _ptr(k), _ptr(v), _ptr(lens),
                                 max_len, n, t, hkv, d, s_cap, _stream(stream)))


def _attn_shapes(q, k, v, cache_k, cache_v):
    n, t, hq, d = q.shape
    hkv = k.shape[2]
    s_cap = cache_k.shape[2]
    _f16("q", q)
    _f16("k", k, (n, t, hkv, d))
    _f16("v", v, (n, t, hkv, d))
    _f16("cache_k", cache_k, (n, hkv, s_cap, d))
    _f16("cache_v", cache_v, (n, hkv, s_cap, d))
    return n, t, hq, hkv, d, s_cap


def prefill(q, k, v, positions, cache_k, cache_v, rope: RopeParams, scale: Optional[float] = None,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block without history: rows [0, t) of the caches are written."""
    n, t, hq, hkv, d, s_cap = _attn_shapes(q, k, v, cache_k, cache_v)
    _i32("positions", positions, (n, t))
    if out is None:
        out = _alloc(stream, lambda: torch.empty_like(q))
    _f16("out", out, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(cache_k),
                              _ptr(cache_v), _ptr(out), n, t, hq, hkv, d, s_cap, float(scale),
                              ctypes.byref(rope), _stream(stream)))
    return out


def prefill_kv(q, k, v, positions, cache_k, cache_v, hist_lens, max_hist: int, rope: RopeParams,
               scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Chunked prefill over the history rows [0, hist_lens[u]) of each cache."""
    n, t, hq, hkv, d, s_cap = _attn_shapes(q, k, v, cache_k, cache_v)
    _i32("positions", positions, (n, t))
    _i32("hist_lens", hist_lens, (n,))
    if out is None:
        out = _alloc(stream, lambda: torch.empty_like(q))
    _f16("out", out, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().attn_prefill_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(cache_k),
                                 _ptr(cache_v), _ptr(hist_lens), int(max_hist), _ptr(out), n, t,
                                 hq, hkv, d, s_cap, float(scale), ctypes.byref(rope),
                                 _stream(stream)))
    return out


def prefill_kv_varlen(q, k, v, positions, cache_k, cache_v, hist_lens, new_lens, max_hist: int,
                      rope: RopeParams, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """prefill_kv where unit u brings new_lens[u] <= t new tokens (rows past it are padding:
    not appended, their out rows left as they were)."""
    n, t, hq, hkv, d, s_cap = _attn_shapes(q, k, v, cache_k, cache_v)
    _i32("positions", positions, (n, t))
    _i32("hist_lens", hist_lens, (n,))
    _i32("new_lens", new_lens, (n,))
    if out is None:
        out = _alloc(stream, lambda: torch.zeros_like(q))
    _f16("out", out, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().attn_prefill_kv_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(cache_k),
                                        _ptr(cache_v), _ptr(hist_lens), int(max_hist), _ptr(new_lens),
                                        _ptr(out), n, t, hq, hkv, d, s_cap, float(scale),
                                        ctypes.byref(rope), _stream(stream)))
    return out


def _weights(w: torch.Tensor, n: int, rows: int, cols: int, name: str) -> int:
    """w [rows, cols] (shared) or [n, rows, cols] (one per unit); returns w_per_unit."""
    per_unit = 1 if w.dim() == 3 else 0
    _f16(name, w, (n, rows, cols) if per_unit else (rows, cols))
    return per_unit


def qkv_project(x, w_qkv, positions, cache_k, cache_v, lens, max_len: int, rope: RopeParams, hq: int,
                hkv: int, q_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Fused QKV projection: returns q [n, t, hq, 128] (unrotated); k (rotated) and v go
    to cache rows lens[u] + i.  x [n, t, hidden]; w_qkv [(hq + 2 hkv) * 128, hidden] or one
    such matrix per unit [n, ...]."""
    if x.dim() != 3:
        raise ValueError("x must be [n, t, hidden]")
    n, t, hidden = x.shape
    d = 128
    _f16("x", x, (n, t, hidden))
    per_unit = _weights(w_qkv, n, (hq + 2 * hkv) * d, hidden, "w_qkv")
    s_cap = cache_k.shape[2]
    _f16("cache_k", cache_k, (n, hkv, s_cap, d))
    _f16("cache_v", cache_v, (n, hkv, s_cap, d))
    _i32("positions", positions, (n, t))
    if lens is not None:
        _i32("lens", lens, (n,))
    if q_out is None:
        q_out = _alloc(stream, lambda: torch.empty((n, t, hq, d), dtype=torch.float16, device=x.device))
    _f16("q_out", q_out, (n, t, hq, d))
    _check(lib().attn_qkv_project(_ptr(x), _ptr(w_qkv), per_unit, _ptr(positions), _ptr(q_out),
                                  _ptr(cache_k), _ptr(cache_v), _ptr(lens) if lens is not None else None,
                                  int(max_len), n, t, hidden, hq, hkv, d, s_cap, ctypes.byref(rope),
                                  _stream(stream)))
    return q_out


def prefill_kv_cached(q, positions, cache_k, cache_v, hist_lens, max_hist: int, rope: RopeParams,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """prefill_kv over caches that already hold the new rows (from qkv_project)."""
    n, t, hq, d = q.shape
    _f16("q", q, (n, t, hq, d))
    hkv, s_cap = cache_k.shape[1], cache_k.shape[2]
    _f16("cache_k", cache_k, (n, hkv, s_cap, d))
    _f16("cache_v", cache_v, (n, hkv, s_cap, d))
    _i32("positions", positions, (n, t))
    if hist_lens is not None:
        _i32("hist_lens", hist_lens, (n,))
    if out is None:
        out = _alloc(stream, lambda: torch.empty_like(q))
    _f16("out", out, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().attn_prefill_kv_cached(_ptr(q), _ptr(positions), _ptr(cache_k), _ptr(cache_v),
                                        _ptr(hist_lens) if hist_lens is not None else None, int(max_hist),
                                        _ptr(out), n, t, hq, hkv, d, s_cap, float(scale), ctypes.byref(rope),
                                        _stream(stream)))
    return out


def out_project(attn, w_o, residual, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out = attn . w_o^T + residual.  attn [n, t, hq, 128]; w_o [hidden, hq * 128] or
    [n, hidden, hq * 128]; residual [n, t, hidden]."""
    if attn.dim() != 4:
        raise ValueError("attn must be [n, t, hq, 128]")
    n, t, hq, d = attn.shape
    _f16("attn", attn, (n, t, hq, d))
    if residual.dim() != 3:
        raise ValueError("residual must be [n, t, hidden]")
    hidden = residual.shape[2]
    _f16("residual", residual, (n, t, hidden))
    per_unit = _weights(w_o, n, hidden, hq * d, "w_o")
    if out is None:
        out = _alloc(stream, lambda: torch.empty_like(residual))
    _f16("out", out, (n, t, hidden))
    _check(lib().attn_out_project(_ptr(attn), _ptr(w_o), per_unit, _ptr(residual), _ptr(out), n, t, hq, d,
                                  hidden, _stream(stream)))
    return out


def decode(q, k, v, positions, cache_k, cache_v, lens, max_len: int, rope: RopeParams,
           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step.  q [n, 1, hq, 128] (or [n, hq, 128]); k, v [n, 1, hkv, 128];
    positions [n] (or [n, 1]); the new rows go to cache row lens[u]."""
    if q.dim() == 3:
        q = q.unsqueeze(1)
    if k.dim() == 3:
        k = k.unsqueeze(1)
    if v.dim() == 3:
        v = v.unsqueeze(1)
    n, t, hq, hkv, d, s_cap = _attn_shapes(q, k, v, cache_k, cache_v)
    if t != 1:
        raise ValueError("decode takes exactly one new token per unit")
    positions = positions.reshape(n)
    _i32("positions", positions, (n,))
    _i32("lens", lens, (n,))
    if out is None:
        out = _alloc(stream, lambda: torch.empty_like(q))
    _f16("out", out, q.shape)
    need = workspace_size(n, hq, hkv, max_len, d)
    if workspace is None:
        workspace = _alloc(stream, lambda: torch.empty(max(need, 16), dtype=torch.uint8, device=q.device))
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 CUDA tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(cache_k),
                             _ptr(cache_v), _ptr(lens), int(max_len), _ptr(out), n, hq, hkv, d,
                             s_cap, float(scale), ctypes.byref(rope), _ptr(workspace),
                             workspace.numel(), _stream(stream)))
    return out
