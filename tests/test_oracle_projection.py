"""Pins for the oracle's projections (Sophgo paper, sec. 3.1 Listings 1-2: q, k, v =
MatMul(x, w), h = Add(input, MatMul(attn, w_o))): a pure-Python dot product on tiny shapes,
exactness where the result is representable, the fused-weight split into q / k / v, the
per-unit weights, and the residual of the output projection (a zero weight returns it bit
for bit; exact integer sums add it once), with mutants the residual pins must catch."""
import inspect
import textwrap
import types

import numpy as np
import pytest


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


def test_per_unit_weights_equal_a_shared_weight(ora):
    rng = np.random.default_rng(53)
    n, t, f, hidden = 3, 5, 16, 8
    attn = _f16(rng.standard_normal((n, t, f)))
    w = _f16(rng.standard_normal((n, hidden, f)))
    res = _f16(rng.standard_normal((n, t, hidden)))
    # per-unit weights: unit u uses w[u] (a unit alone with its matrix as the shared one)
    yp, _ = ora.out_project(attn, w, res)
    for u in range(n):
        yu, _ = ora.out_project(attn[u:u + 1], w[u], res[u:u + 1])
        assert np.array_equal(yp[u], yu[0])
    # shared weights = per-unit weights all equal to it
    ys, _ = ora.out_project(attn, w[0], res)
    yq, _ = ora.out_project(attn, np.stack([w[0]] * n), res)
    assert np.array_equal(ys, yq)


def test_zero_weight_returns_the_residual_bit_for_bit(ora):
    # Add(input, MatMul(attn, w_o)) with w_o = 0: the block's output is its input exactly
    rng = np.random.default_rng(54)
    n, t, f, hidden = 2, 7, 32, 16
    attn = _f16(rng.standard_normal((n, t, f)))
    res = _f16(rng.standard_normal((n, t, hidden)) * 3)
    y64, y16 = ora.out_project(attn, np.zeros((hidden, f), np.uint16), res)
    assert np.array_equal(y16, res)
    assert np.array_equal(y64, res.view(np.float16).astype(np.float64))


def test_residual_is_added_once_on_exact_integers(ora):
    # integer-valued f16 operands whose products, sums and residual stay below 2^11: the
    # block's output is the exact integer attn . w_o^T + residual, computed here in int64
    rng = np.random.default_rng(55)
    n, t, f, hidden = 2, 6, 24, 10
    a = rng.integers(-3, 4, (n, t, f))
    w = rng.integers(-3, 4, (hidden, f))
    r = rng.integers(-400, 401, (n, t, hidden))
    ref = np.einsum("ntf,hf->nth", a, w) + r
    assert np.abs(ref).max() < 2048
    y64, y16 = ora.out_project(_f16(a), _f16(w), _f16(r))
    assert np.array_equal(y64, ref.astype(np.float64))
    assert np.array_equal(y16.view(np.float16).astype(np.int64), ref)


RESIDUAL_PINS = [test_zero_weight_returns_the_residual_bit_for_bit,
                 test_residual_is_added_once_on_exact_integers]


@pytest.mark.parametrize("mutation", ["y = y", "y = y + 2.0 * f16_to_f64(res)", "y = y - f16_to_f64(res)"])
def test_residual_pins_catch_planted_mistakes(ora, mutation):
    """A copy of out_project with the residual dropped, doubled or subtracted: the pins
    above must reject it (the projection helpers are Python, so the mistake is planted in
    a copy of that function's source)."""
    src = textwrap.dedent(inspect.getsource(ora.out_project))
    site = "y = y + f16_to_f64(res)"
    assert src.count(site) == 1
    mut = types.ModuleType("oracle_mutant")
    mut.__dict__.update(ora.__dict__)
    exec(compile(src.replace(site, mutation), "<mutant>", "exec"), mut.__dict__)
    caught = 0
    for pin in RESIDUAL_PINS:
        try:
            pin(mut)
        except AssertionError:
            caught += 1
    assert caught == len(RESIDUAL_PINS)
