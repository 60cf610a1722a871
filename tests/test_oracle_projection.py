"""Pins for the oracle's projections (Sophgo paper, sec. 3.1 Listings 1-2: q, k, v =
MatMul(x, w), h = Add(input, MatMul(attn, w_o))): a pure-Python dot product on tiny shapes,
exactness where the result is representable, the fused-weight split into q / k / v and the
per-unit weights."""
import numpy as np


def _f16(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def test_projection_matches_brute_force_dot_products(ora):
    rng = np.random.default_rng(50)
    a = rng.standard_normal((3, 4, 24)).astype(np.float16)
    w = rng.standard_normal((5, 24)).astype(np.float16)
    y64, y16 = ora.project(_f16(a).reshape(12, 24), _f16(w))
    for r in range(12):
        for c in range(5):
            s = 0.0
            for kk in range(24):
                s += float(a.reshape(12, 24)[r, kk]) * float(w[c, kk])
            assert abs(y64[r, c] - s) <= 1e-12 * max(1.0, abs(s))
    assert np.array_equal(y16, ora.f64_to_f16(y64))


def test_projection_is_exact_on_small_integers(ora):
    # integer-valued f16 inputs: every dot product is an integer below 2^11, exact in f16
    rng = np.random.default_rng(51)
    a = rng.integers(-3, 4, (6, 32)).astype(np.float16)
    w = rng.integers(-3, 4, (7, 32)).astype(np.float16)
    y64, y16 = ora.project(_f16(a), _f16(w))
    ref = a.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(y64, ref.astype(np.float64))
    assert np.array_equal(y16.view(np.float16).astype(np.int64), ref)


def test_qkv_split_selects_rows_of_the_fused_weight(ora):
    # a selection weight (one 1 per row) copies input features: q / k / v land in the
    # right heads and dims
    n, t, hidden, hq, hkv, d = 2, 3, 64, 2, 1, 8
    rng = np.random.default_rng(52)
    x = rng.standard_normal((n, t, hidden)).astype(np.float16)
    rows = (hq + 2 * hkv) * d
    sel = rng.integers(0, hidden, rows)
    w = np.zeros((rows, hidden), np.float16)
    w[np.arange(rows), sel] = 1.0
    q, k, v = ora.qkv_project(_f16(x), _f16(w), hq, hkv, d)
    y = x[..., sel]
    assert np.array_equal(q.view(np.float16), y[..., : hq * d].reshape(n, t, hq, d))
    assert np.array_equal(k.view(np.float16), y[..., hq * d: (hq + hkv) * d].reshape(n, t, hkv, d))
    assert np.array_equal(v.view(np.float16), y[..., (hq + hkv) * d:].reshape(n, t, hkv, d))


def test_per_unit_weights_and_residual(ora):
    rng = np.random.default_rng(53)
    n, t, f, hidden = 3, 5, 16, 8
    attn = _f16(rng.standard_normal((n, t, f)))
    w = _f16(rng.standard_normal((n, hidden, f)))
    res = _f16(rng.standard_normal((n, t, hidden)))
    y64, y16 = ora.out_project(attn, w, res)
    for u in range(n):
        a64, w64, r64 = (ora.f16_to_f64(z[u]) for z in (attn, w, res))
        np.testing.assert_allclose(y64[u], a64 @ w64.T + r64, rtol=0, atol=1e-13)
    # shared weights = per-unit weights all equal to it
    ys, _ = ora.out_project(attn, w[0], res)
    yp, _ = ora.out_project(attn, np.stack([w[0]] * n), res)
    assert np.array_equal(ys, yp)
