"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (written here, used by every parity test):
  * attention outputs (f16, fp32 accumulation on the GPU) against the oracle's unrounded
    fp64 output: max |gpu - ref| <= 2e-3 and, per (unit, token, head) row,
    max_d |gpu - ref| / max_d |ref| <= 1e-2;
  * cache rows: V rows and untouched rows bit-identical; rotated K rows equal to the
    oracle's f16 rounding of its fp64 rotation.  A K element may differ only when the
    exact value sits on an f16 rounding boundary within what fp64 trig can resolve: the
    oracle's fp64 value is within 1e-11 (relative to max(1, |value|)) of the midpoint of
    the two candidates and the GPU took the other neighbour.  The band covers the two
    sides' angle evaluations: each rounds the product position x frequency once (under
    4e-12 rad at positions below 2^15) and the GPU's sin / cos series stays within 1e-16
    of the exact values, so |x| x 7e-12 bounds the difference of the rotated values.
    Such cases are counted and expected to be (nearly) zero.
"""
import numpy as np
import torch

ATOL = 2e-3
ROW_RTOL = 1e-2
K_BAND = 1e-11


def to_np_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return b.view(np.float16).astype(np.float64)


def check_attention(gpu_bits: np.ndarray, ref64: np.ndarray, what: str = "out"):
    """gpu_bits: f16 bits [..., d]; ref64: fp64 [..., d]."""
    g = bits_to_f64(gpu_bits)
    assert g.shape == ref64.shape, (g.shape, ref64.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - ref64)
    max_abs = float(err.max()) if err.size else 0.0
    denom = np.maximum(np.abs(ref64).max(axis=-1), 1e-30)
    row_rel = float((err.max(axis=-1) / denom).max()) if err.size else 0.0
    assert max_abs <= ATOL, f"{what}: max abs error {max_abs:.3e} > {ATOL}"
    assert row_rel <= ROW_RTOL, f"{what}: row-relative error {row_rel:.3e} > {ROW_RTOL}"
    return max_abs, row_rel


def error_profile(gpu_bits: np.ndarray, ref64: np.ndarray) -> dict:
    """Where the largest error sits: its index and the reference magnitude there."""
    g = bits_to_f64(gpu_bits)
    err = np.abs(g - ref64)
    if not err.size:
        return {"ref_at_max_abs": 0.0, "where": None}
    i = int(np.argmax(err))
    return {"ref_at_max_abs": float(np.abs(ref64.reshape(-1)[i])),
            "where": tuple(int(x) for x in np.unravel_index(i, err.shape))}


def check_k_rows(gpu_bits: np.ndarray, ref_bits: np.ndarray, ref64: np.ndarray, what="k"):
    """Rotated K rows: bit-exact except on an fp64-unresolvable rounding boundary."""
    mism = gpu_bits != ref_bits
    n_bad = int(mism.sum())
    if n_bad:
        g = bits_to_f64(gpu_bits[mism])
        o = bits_to_f64(ref_bits[mism])
        v = ref64[mism]
        mid = (g + o) / 2
        ok = np.abs(v - mid) <= K_BAND * np.maximum(1.0, np.abs(v))
        # the two candidates must be adjacent f16 values
        gi = gpu_bits[mism].astype(np.int32)
        oi = ref_bits[mism].astype(np.int32)
        adjacent = np.abs(gi - oi) == 1
        bad = ~(ok & adjacent)
        assert not bad.any(), (f"{what}: {int(bad.sum())} rotated K values differ from the "
                               f"oracle's rounding (of {mism.size})")
    return n_bad
