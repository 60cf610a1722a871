"""Binding of libkvrope_probes.so (include/kvrope_probes.h): the measurement helpers a
benchmark reports beside the spec peaks, and the kernels' f16 rounding compiled for the
host.  Not part of the attention path."""
from __future__ import annotations

import ctypes
import os

import torch  # first: the library binds to the HIP runtime torch has loaded

from . import HERE, KVRopeError, ATTN_OK, _ptr, _stream, status_string

LIB_PATH = os.path.join(HERE, "libkvrope_probes.so")
EXPORTS = ["kvprobe_read", "kvprobe_stream", "kvprobe_mfma", "kvprobe_f64_to_f16"]

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m kv_cache_causal_rope_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kvprobe_read.argtypes = [_P, ctypes.c_size_t, _I, _P, _P]
        L.kvprobe_stream.argtypes = [_P, _P, _P] + [_I] * 6 + [_P, _P]
        L.kvprobe_mfma.argtypes = [_I, _I, _P, _P]
        for f in ("kvprobe_read", "kvprobe_stream", "kvprobe_mfma"):
            getattr(L, f).restype = _I
        L.kvprobe_f64_to_f16.argtypes = [ctypes.c_double]
        L.kvprobe_f64_to_f16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise KVRopeError(status, status_string(status))


def f64_to_f16_bits(x: float) -> int:
    """The kernels' fp64 -> f16 conversion, run on the host (for tests)."""
    return int(lib().kvprobe_f64_to_f16(float(x)))


def read(buf: torch.Tensor, blocks: int, sink: torch.Tensor, stream=None):
    """Read all of `buf` (contiguous CUDA tensor, a multiple of 16 bytes) once."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().kvprobe_read(_ptr(buf), nbytes, int(blocks), _ptr(sink), _stream(stream)))


def stream_rows(cache_k, cache_v, lens, max_len: int, chunk: int, sink, stream=None):
    """Read (only) rows [0, lens[u]] of every (unit, KV head) of the caches, in chunks of
    `chunk` rows per workgroup."""
    n, hkv, s_cap, d = cache_k.shape
    _check(lib().kvprobe_stream(_ptr(cache_k), _ptr(cache_v), _ptr(lens), n, hkv, s_cap, d, int(max_len),
                                int(chunk), _ptr(sink), _stream(stream)))


def mfma(blocks: int, iters: int, sink, stream=None):
    """`blocks` workgroups x 4 waves, each `iters` rounds of 4 independent f16 MFMAs
    (32x32x16); sink (uint64) gets per-workgroup clock counters at [4 + 4b, 8 + 4b)."""
    _check(lib().kvprobe_mfma(int(blocks), int(iters), _ptr(sink), _stream(stream)))
