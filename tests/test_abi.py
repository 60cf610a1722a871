"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every function include/kvrope.h declares, and every
host-decided status must come back before any HIP call -- these tests pass fake but
aligned device pointers, which the library never dereferences on the host.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvrope.h")
PROBES_HEADER = os.path.join(ROOT, "include", "kvrope_probes.h")


@pytest.fixture(scope="module")
def kv():
    import kv_cache_causal_rope_amd as kv
    if not os.path.exists(kv.LIB_PATH):
        from kv_cache_causal_rope_amd import build
        build.build()
    kv.lib()
    return kv


def _declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_the_scope_table_boundary():
    # the five entry points, the workspace query and the status strings, under the names
    # of the boundary the build was planned against
    names = _declared_functions()
    for ep in ["attn_rope_apply", "kv_cache_append", "attn_prefill", "attn_prefill_kv",
               "attn_decode", "attn_workspace_size", "attn_status_string"]:
        assert ep in names
    src = open(HEADER).read()
    for code in ["ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_ROPE", "ATTN_ERR_CAPACITY",
                 "ATTN_ERR_ALIGN", "ATTN_ERR_WORKSPACE", "ATTN_ERR_HIP"]:
        assert re.search(r"#define\s+%s\b" % code, src), code


def test_library_exports_every_declared_symbol(kv):
    exported = _exported(kv.LIB_PATH)
    declared = _declared_functions()
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    assert sorted(kv.EXPORTS) == declared


def test_measurement_helpers_are_outside_the_product_library(kv):
    from kv_cache_causal_rope_amd import probes
    product = {n for n in _exported(kv.LIB_PATH) if n.startswith(("attn_", "kv_", "kvprobe_", "kvrope_"))}
    assert product == set(kv.EXPORTS), sorted(product ^ set(kv.EXPORTS))
    declared = _declared_functions(PROBES_HEADER)
    assert sorted(probes.EXPORTS) == declared
    missing = [n for n in declared if n not in _exported(probes.LIB_PATH)]
    assert not missing, missing


def test_single_hip_runtime_in_process(kv):
    assert kv._count_hip_runtimes() <= 1


# fake, 16-byte aligned "device" pointers: never dereferenced on the host
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
UNALIGNED = ctypes.c_void_p(0x10008)


def _prefill_kv(kv, **over):
    args = dict(q=A, k=A, v=A, pos=A, hk=B, hv=B, hl=A, max_hist=10, out=B, n=2, t=4, hq=12,
                hkv=2, d=128, s_cap=20, scale=0.088, rp=kv.RopeParams.plain(), stream=None)
    args.update(over)
    rp = args["rp"]
    return kv.lib().attn_prefill_kv(args["q"], args["k"], args["v"], args["pos"], args["hk"],
                                    args["hv"], args["hl"], args["max_hist"], args["out"],
                                    args["n"], args["t"], args["hq"], args["hkv"], args["d"],
                                    args["s_cap"], args["scale"],
                                    ctypes.byref(rp) if rp is not None else None, args["stream"])


@pytest.mark.parametrize("over,expect", [
    (dict(d=64), -2), (dict(hq=7), -2), (dict(hkv=0), -2), (dict(n=-1), -2),
    (dict(s_cap=0), -2),
    (dict(q=None), -1), (dict(out=None), -1), (dict(hk=None), -1), (dict(rp=None), -1),
    (dict(q=UNALIGNED), -5), (dict(hv=UNALIGNED), -5),
    (dict(max_hist=17), -4), (dict(max_hist=-1), -4),
    (dict(scale=0.0), -7), (dict(scale=float("nan")), -7), (dict(scale=float("inf")), -7),
])
def test_prefill_kv_host_validation(kv, over, expect):
    assert _prefill_kv(kv, **over) == expect


@pytest.mark.parametrize("field,value", [
    ("n_rot", 3), ("n_rot", 0), ("n_rot", 130), ("base", 1.0), ("base", float("nan")),
    ("mscale", 0.0), ("yarn", 2),
])
def test_rope_parameter_validation(kv, field, value):
    rp = kv.RopeParams.plain()
    setattr(rp, field, value)
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE


@pytest.mark.parametrize("field,value", [
    ("freq_scale", 0.0), ("ext_factor", 1.5), ("n_ctx_orig", 0), ("beta_fast", -1.0),
    ("beta_slow", float("inf")),
])
def test_yarn_parameter_validation(kv, field, value):
    rp = kv.RopeParams.yarn_tail()
    setattr(rp, field, value)
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE


def test_zero_sized_calls_are_noops(kv):
    assert _prefill_kv(kv, n=0) == 0
    assert _prefill_kv(kv, t=0) == 0
    L = kv.lib()
    assert L.attn_prefill(None, None, None, None, None, None, None, 0, 5, 12, 2, 128, 8, 0.1,
                          ctypes.byref(kv.RopeParams.plain()), None) == 0


def test_prefill_without_history_checks_capacity(kv):
    L = kv.lib()
    rp = kv.RopeParams.plain()
    assert L.attn_prefill(A, A, A, A, B, B, B, 1, 9, 12, 2, 128, 8, 0.1, ctypes.byref(rp), None) == -4


def test_decode_validation_and_workspace(kv):
    L = kv.lib()
    rp = kv.RopeParams.plain()
    n, hq, hkv, max_len, s_cap = 28, 12, 2, 1024, 1025
    need = kv.workspace_size(n, hq, hkv, max_len)
    assert need > 0 and need % 4 == 0

    def call(ws=A, ws_bytes=need, max_len=max_len, s_cap=s_cap, hq=hq, lens=A):
        return L.attn_decode(A, A, A, A, B, B, lens, max_len, B, n, hq, hkv, 128, s_cap, 0.088,
                             ctypes.byref(rp), ws, ws_bytes, None)

    assert call(ws=None) == kv.ATTN_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == kv.ATTN_ERR_WORKSPACE
    assert call(ws=UNALIGNED) == kv.ATTN_ERR_ALIGN
    assert call(s_cap=1024) == kv.ATTN_ERR_CAPACITY
    assert call(hq=13) == kv.ATTN_ERR_SHAPE
    assert call(lens=None) == kv.ATTN_ERR_NULL
    assert L.attn_workspace_size(kv.ATTN_OP_DECODE, n, 1, 13, 2, 128, 10) == 0


def test_decode_split_sizes(kv):
    """The decode split (host arithmetic only): chunks of 256 to 1024 keys, a multiple of
    32, about two workgroups' worth per compute unit; the workspace holds one partial per
    (unit, head, chunk) of the longest cache."""
    for n, hq, hkv, max_len, expect in [(28, 12, 2, 1024, 256),      # one sequence, rows to 1024
                                        (28, 12, 2, 4095, 448),      # rows to 4096
                                        (896, 12, 2, 4096, 1024),    # 28 layers x batch 32
                                        (256, 64, 8, 32768, 1024),   # YaRN 32k batch 64
                                        (1, 8, 8, 10, 256)]:
        chunk = kv.decode_chunk_keys(n, hq, hkv, max_len)
        assert chunk == expect, (n, hq, hkv, max_len, chunk)
        assert 256 <= chunk <= 1024 and chunk % 32 == 0
        nsplit = (max_len + 1 + chunk - 1) // chunk
        assert kv.workspace_size(n, hq, hkv, max_len) == n * hq * nsplit * 130 * 4


def test_append_and_rope_validation(kv):
    L = kv.lib()
    rp = kv.RopeParams.plain()
    assert L.kv_cache_append(B, B, A, A, A, 5, 2, 4, 2, 128, 8, None) == kv.ATTN_ERR_CAPACITY
    assert L.kv_cache_append(B, B, A, A, None, 4, 2, 4, 2, 128, 8, None) == kv.ATTN_ERR_NULL
    assert L.kv_cache_append(B, B, UNALIGNED, A, A, 4, 2, 4, 2, 128, 8, None) == kv.ATTN_ERR_ALIGN
    assert L.kv_cache_append(B, B, A, A, A, 4, 2, 4, 2, 96, 8, None) == kv.ATTN_ERR_SHAPE
    assert L.attn_rope_apply(A, A, 2, 3, 4, 120, ctypes.byref(rp), None) == kv.ATTN_ERR_SHAPE
    assert L.attn_rope_apply(None, A, 2, 3, 4, 128, ctypes.byref(rp), None) == kv.ATTN_ERR_NULL
    assert L.attn_rope_apply(A, A, 0, 3, 4, 128, ctypes.byref(rp), None) == 0


def test_status_strings(kv):
    for code in range(-8, 1):
        assert kv.status_string(code)
    assert kv.status_string(-99) == "unknown status"


def test_kernel_f16_conversion_on_host(kv):
    """The fp64 -> f16 conversion the kernels use for rotated K, against numpy."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(5000) * 1e-5,
                        rng.standard_normal(5000) * 3e4, [65504.0, 65519.99, 65520.0, 2.0 ** -25,
                                                          np.nextafter(2.0 ** -25, 1), -0.0, 0.0,
                                                          np.inf, -np.inf]])
    # exact midpoints between adjacent f16 values
    lo = np.arange(0, 0x7bff, 97, dtype=np.uint16)
    a = lo.view(np.float16).astype(np.float64)
    b = (lo + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (a + b) / 2, -(a + b) / 2])
    from kv_cache_causal_rope_amd import probes
    got = np.array([probes.f64_to_f16_bits(v) for v in x], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    nan = probes.f64_to_f16_bits(float("nan"))
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


@pytest.mark.parametrize("field,value", [("pairing", 2), ("pairing", -1), ("inverse", 2)])
def test_rotation_variant_validation(kv, field, value):
    rp = kv.RopeParams.plain()
    setattr(rp, field, value)
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE


@pytest.mark.parametrize("n_rot", [2, 16, 48, 100])
def test_half_split_needs_a_multiple_of_32(kv, n_rot):
    rp = kv.RopeParams.plain(n_rot=n_rot)
    rp.pairing = 1
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE


def test_table_validation(kv):
    rp = kv.RopeParams.plain()
    rp.cos_table, rp.sin_table, rp.table_rows = A.value, None, 10
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE          # one table without the other
    rp.sin_table, rp.table_rows = A.value, 0
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE          # no rows
    rp.table_rows, rp.sin_table = 10, 0x10002
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ALIGN         # misaligned float table


def test_varlen_host_validation(kv):
    L = kv.lib()
    rp = ctypes.byref(kv.RopeParams.plain())
    args = [A, A, A, A, B, B, A, 10]
    # NULL new-token counts, misaligned counts, zero-sized call
    assert L.attn_prefill_kv_varlen(*args, None, B, 2, 4, 12, 2, 128, 20, 0.088, rp, None) == -1
    assert L.attn_prefill_kv_varlen(*args, ctypes.c_void_p(0x10002), B, 2, 4, 12, 2, 128, 20, 0.088, rp,
                                    None) == -5
    assert L.attn_prefill_kv_varlen(*args, None, B, 0, 4, 12, 2, 128, 20, 0.088, rp, None) == 0
    assert L.attn_prefill_kv_varlen(*args, A, B, 2, 4, 12, 2, 128, 13, 0.088, rp, None) == -4


def test_projection_host_validation(kv):
    L = kv.lib()
    rp = ctypes.byref(kv.RopeParams.plain())
    # x, w, w_per_unit, pos, q, ck, cv, lens, max_len, n, t, hidden, hq, hkv, d, s_cap
    ok = [A, A, 0, A, B, B, B, A, 4, 2, 8, 256, 12, 2, 128, 16]
    def qkv(**over):
        args = list(ok)
        for i, val in over.items():
            args[int(i[1:])] = val
        return L.attn_qkv_project(*args, rp, None)
    assert qkv(a11=100) == -2          # hidden not a multiple of 64
    assert qkv(a2=2) == -2             # w_per_unit not 0/1
    assert qkv(a14=64) == -2           # head dim
    assert qkv(a0=None) == -1
    assert qkv(a4=UNALIGNED) == -5
    assert qkv(a15=11) == -4           # max_len + t > s_cap
    assert qkv(a9=0) == 0              # nothing to do
    # attn, w_o, w_per_unit, residual, out, n, t, hq, d, hidden
    assert L.attn_out_project(A, A, 0, A, B, 2, 8, 12, 128, 100, None) == -2   # hidden % 128
    assert L.attn_out_project(A, None, 0, A, B, 2, 8, 12, 128, 256, None) == -1
    assert L.attn_out_project(A, A, 0, UNALIGNED, B, 2, 8, 12, 128, 256, None) == -5
    assert L.attn_out_project(A, A, 0, A, B, 0, 8, 12, 128, 256, None) == 0
    # q, pos, ck, cv, hist, max_hist, out, n, t, hq, hkv, d, s_cap, scale
    assert L.attn_prefill_kv_cached(A, A, B, B, A, 4, B, 2, 8, 12, 2, 128, 11, 0.1, rp, None) == -4
    assert L.attn_prefill_kv_cached(A, A, B, B, A, 4, B, 2, 8, 12, 2, 128, 16, 0.0, rp, None) == -7
    assert L.attn_prefill_kv_cached(None, A, B, B, A, 4, B, 2, 8, 12, 2, 128, 16, 0.1, rp, None) == -1


def test_parameter_set_validation(kv):
    import torch
    plain, yarn = kv.RopeParams.plain(), kv.RopeParams.yarn_tail(n_rot=128)
    us = torch.zeros(2, dtype=torch.int32)          # host memory: never dereferenced here
    rp = kv.RopeParams.plain()
    arr = (kv.RopeParams * 2)(plain, yarn)
    rp.n_sets, rp.sets, rp.unit_set = 2, ctypes.cast(arr, ctypes.POINTER(kv.RopeParams)), A.value
    assert _prefill_kv(kv, rp=rp, n=0) == 0
    rp.n_sets = kv.MAX_ROPE_SETS + 1
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE                 # too many sets
    rp.n_sets = -1
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE
    rp.n_sets = 2
    arr[1].ext_factor = 2.0
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE                 # a bad set
    arr[1].ext_factor = 1.0
    rp.unit_set = 0x10002
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ALIGN                # misaligned indices
    rp.unit_set = None
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_NULL                 # no indices
    rp.unit_set = A.value
    rp.sets = None
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_NULL                 # no sets
    rp.sets = ctypes.cast(arr, ctypes.POINTER(kv.RopeParams))
    rp.cos_table, rp.sin_table, rp.table_rows = A.value, A.value, 10
    assert _prefill_kv(kv, rp=rp) == kv.ATTN_ERR_ROPE                 # sets and tables
    # the outer struct's own frequency fields are not read when sets are given
    rp.cos_table = rp.sin_table = None
    rp.table_rows, rp.base = 0, 0.5
    assert _prefill_kv(kv, rp=rp, n=0) == 0
    del us

