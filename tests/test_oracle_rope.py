"""Pins for the oracle's rotary embedding (plain and YaRN tail rotation).

What the pages fix (ds4.c study notes, Part 4 sec. 1, Traces 1-2):
  * a pair (x0, x1) is multiplied by [[cos t, -sin t], [sin t, cos t]];
  * t = pos * base^(-2j/n_rot) for pair j; position 0 is no rotation;
  * rotation encodes relative position: <R(m) q, R(n) k> depends on m - n only;
  * the YaRN ramp is 1 below the fast correction dim and 0 above the slow one; the
    correction dim is where a pair turns beta full circles over the original context.
Each test checks one of these from outside the formula (textbook constants, norms,
shifts, an independent complex-number route, limiting cases), so a dropped term, a sign
flip or a wrong exponent in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "circular_functions.json")))


def _f16(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def _rand_f16(rng, shape):
    return rng.standard_normal(shape).astype(np.float16).view(np.uint16)


def test_position_zero_is_identity_bit_exact(ora):
    rng = np.random.default_rng(0)
    x = _rand_f16(rng, (7, 3, 128))
    out, out64 = ora.rope(x, np.zeros(7, np.int32), ora.RopeParams.plain())
    assert np.array_equal(out, x)
    assert np.array_equal(out64, ora.f16_to_f64(x))


def test_pair0_turns_by_position_radians_textbook(ora):
    # omega_0 = base^0 = 1: pair 0 at pos p turns by exactly p radians.
    x = np.zeros((3, 1, 128), np.float16)
    x[:, 0, 0] = 1.0        # (1, 0) -> (cos p, sin p)
    x[:, 0, 3] = 1.0        # pair 1 = (0, 1) -> rotated, ignored here
    pos = np.array([1, 2, 0], np.int32)
    _, y = ora.rope(_f16(x), pos, ora.RopeParams.plain())
    assert y[0, 0, 0] == pytest.approx(GOLD["cos_1"], abs=1e-15)
    assert y[0, 0, 1] == pytest.approx(GOLD["sin_1"], abs=1e-15)
    assert y[1, 0, 0] == pytest.approx(GOLD["cos_2"], abs=1e-15)
    assert y[1, 0, 1] == pytest.approx(GOLD["sin_2"], abs=1e-15)
    # direction: (0, 1) -> (-sin, cos)
    x2 = np.zeros((1, 1, 128), np.float16)
    x2[0, 0, 1] = 1.0
    _, y2 = ora.rope(_f16(x2), np.array([1], np.int32), ora.RopeParams.plain())
    assert y2[0, 0, 0] == pytest.approx(-GOLD["sin_1"], abs=1e-15)
    assert y2[0, 0, 1] == pytest.approx(GOLD["cos_1"], abs=1e-15)


@pytest.mark.parametrize("pair,pos", [(16, 10), (32, 100), (48, 1000)])
def test_frequency_schedule_textbook(ora, pair, pos):
    # base 1e4, n_rot 128: omega_j = 10^(-j/16), so pair 16 at pos 10, pair 32 at pos 100
    # and pair 48 at pos 1000 all turn by 1 radian.
    x = np.zeros((1, 1, 128), np.float16)
    x[0, 0, 2 * pair] = 1.0
    _, y = ora.rope(_f16(x), np.array([pos], np.int32), ora.RopeParams.plain())
    assert y[0, 0, 2 * pair] == pytest.approx(GOLD["cos_1"], abs=1e-13)
    assert y[0, 0, 2 * pair + 1] == pytest.approx(GOLD["sin_1"], abs=1e-13)
    # every other pair stays zero
    others = np.delete(y[0, 0], [2 * pair, 2 * pair + 1])
    assert np.all(others == 0.0)


def test_tail_half_width_schedule(ora):
    # n_rot = 64 rotates dims [64, 128); its own schedule omega_j = 10^(-j/8):
    # pair 8 of the tail at pos 10 turns by 1 radian.
    x = np.zeros((1, 1, 128), np.float16)
    x[0, 0, 64 + 16] = 1.0
    x[0, 0, 5] = 1.5
    _, y = ora.rope(_f16(x), np.array([10], np.int32), ora.RopeParams.plain(n_rot=64))
    assert y[0, 0, 80] == pytest.approx(GOLD["cos_1"], abs=1e-13)
    assert y[0, 0, 81] == pytest.approx(GOLD["sin_1"], abs=1e-13)
    assert y[0, 0, 5] == 1.5


@pytest.mark.parametrize("rp_name", ["plain", "tail", "yarn"])
def test_pair_norm_scaled_by_mscale_only(ora, rp_name):
    rp = {"plain": ora.RopeParams.plain(), "tail": ora.RopeParams.plain(n_rot=64),
          "yarn": ora.RopeParams.yarn_tail()}[rp_name]
    rng = np.random.default_rng(1)
    x = _rand_f16(rng, (64, 4, 128))
    pos = rng.integers(0, 40000, 64).astype(np.int32)
    _, y = ora.rope(x, pos, rp)
    xd = ora.f16_to_f64(x)
    o = 128 - rp.n_rot
    nx = np.hypot(xd[..., o::2], xd[..., o + 1::2])
    ny = np.hypot(y[..., o::2], y[..., o + 1::2])
    np.testing.assert_allclose(ny, rp.mscale * nx, rtol=1e-14, atol=1e-300)
    # unrotated head dims are copied exactly
    assert np.array_equal(y[..., :o], xd[..., :o])


@pytest.mark.parametrize("rp_name", ["plain", "yarn"])
def test_relative_position_invariance(ora, rp_name):
    rp = ora.RopeParams.plain() if rp_name == "plain" else ora.RopeParams.yarn_tail()
    rng = np.random.default_rng(2)
    qx = _rand_f16(rng, (1, 1, 128))
    kx = _rand_f16(rng, (1, 1, 128))
    base_dots = None
    for shift in [0, 3, 17, 250, 1000]:
        m, n = 37 + shift, 5 + shift
        _, qy = ora.rope(qx, np.array([m], np.int32), rp)
        _, ky = ora.rope(kx, np.array([n], np.int32), rp)
        dot = float(np.dot(qy.ravel(), ky.ravel()))
        if base_dots is None:
            base_dots = dot
        assert dot == pytest.approx(base_dots, rel=1e-11, abs=1e-11)
    # and it does change with the offset m - n
    _, qy = ora.rope(qx, np.array([38], np.int32), rp)
    _, ky = ora.rope(kx, np.array([5], np.int32), rp)
    assert abs(float(np.dot(qy.ravel(), ky.ravel())) - base_dots) > 1e-6


def test_plain_matches_complex_multiplication(ora):
    # independent route: (x0 + i x1) * exp(i pos base^(-2j/n)) in numpy complex128
    rng = np.random.default_rng(3)
    rows = 32
    x = _rand_f16(rng, (rows, 2, 128))
    pos = rng.integers(0, 5000, rows).astype(np.int32)
    _, y = ora.rope(x, pos, ora.RopeParams.plain())
    xd = x.view(np.float16).astype(np.float64)
    z = xd[..., 0::2] + 1j * xd[..., 1::2]
    freqs = np.power(10000.0, -np.arange(64) / 64.0)
    rot = np.exp(1j * pos[:, None, None] * freqs[None, None, :])
    w = z * rot
    np.testing.assert_allclose(y[..., 0::2], w.real, atol=1e-11)
    np.testing.assert_allclose(y[..., 1::2], w.imag, atol=1e-11)


def test_rotated_output_is_rne_of_fp64(ora):
    rng = np.random.default_rng(4)
    x = _rand_f16(rng, (50, 3, 128))
    pos = rng.integers(0, 3000, 50).astype(np.int32)
    out, y = ora.rope(x, pos, ora.RopeParams.yarn_tail())
    assert np.array_equal(out, y.astype(np.float16).view(np.uint16))


# ------------------------------------------------------------------ YaRN
def test_yarn_correction_dims_turn_beta_circles(ora):
    # at the (real-valued) pair index d, a pair of frequency base^(-2d/n_rot) completes
    # n_ctx_orig * omega / (2 pi) turns over the original context: that count is beta.
    rp = ora.RopeParams.yarn_tail()
    _, _, (d0, d1) = ora.rope_freqs(rp)
    turns = lambda d: rp.n_ctx_orig * rp.base ** (-2.0 * d / rp.n_rot) / (2 * math.pi)
    assert turns(d0) == pytest.approx(rp.beta_fast, rel=1e-12)
    assert turns(d1) == pytest.approx(rp.beta_slow, rel=1e-12)
    assert 0 < d0 < d1 < rp.n_rot / 2


def test_yarn_ramp_endpoints_and_linearity(ora):
    rp = ora.RopeParams.yarn_tail()
    _, gamma, (d0, d1) = ora.rope_freqs(rp)
    j = np.arange(rp.n_rot // 2)
    assert np.all(gamma[j < d0] == 1.0)
    assert np.all(gamma[j > d1] == 0.0)
    inner = (j > d0) & (j < d1)
    assert inner.sum() >= 3
    # inner values lie on one line through (d0, 1) and (d1, 0)
    slope, icpt = np.polyfit(j[inner], gamma[inner], 1)
    assert slope * d0 + icpt == pytest.approx(1.0, abs=1e-12)
    assert slope * d1 + icpt == pytest.approx(0.0, abs=1e-12)
    assert np.all(np.diff(gamma) <= 0)
    # the page's ramp helper at its own endpoints
    assert ora.yarn_ramp(2.0, 5.0, 1) == 1.0 and ora.yarn_ramp(2.0, 5.0, 6) == 0.0
    assert ora.yarn_ramp(2.0, 5.0, 3) == pytest.approx(2.0 / 3.0, abs=1e-15)
    # degenerate ramp: denominator floored at 0.001
    assert ora.yarn_ramp(3.0, 3.0, 3) == 1.0 and ora.yarn_ramp(3.0, 3.0, 4) == 0.0


def test_yarn_limits_equal_plain_rotation(ora):
    # gamma = 0 pairs rotate like plain RoPE at pos * freq_scale; gamma = 1 pairs like
    # plain RoPE at pos; both scaled by mscale.
    rp = ora.RopeParams.yarn_tail()
    plain = ora.RopeParams.plain(n_rot=64)
    _, gamma, _ = ora.rope_freqs(rp)
    rng = np.random.default_rng(5)
    x = _rand_f16(rng, (40, 2, 128))
    pos = (rng.integers(0, 8192, 40) * 4).astype(np.int32)
    _, y = ora.rope(x, pos, rp)
    _, y_full = ora.rope(x, pos, plain)
    _, y_quarter = ora.rope(x, pos // 4, plain)
    for jj in range(32):
        sl = slice(64 + 2 * jj, 64 + 2 * jj + 2)
        if gamma[jj] == 0.0:
            ref = y_quarter[..., sl] * rp.mscale
        elif gamma[jj] == 1.0:
            ref = y_full[..., sl] * rp.mscale
        else:
            continue
        np.testing.assert_allclose(y[..., sl], ref, rtol=1e-13, atol=1e-13)
    assert (gamma == 0).sum() > 0 and (gamma == 1).sum() > 0


def test_yarn_position_zero_scales_by_mscale(ora):
    rp = ora.RopeParams.yarn_tail()
    rng = np.random.default_rng(6)
    x = _rand_f16(rng, (3, 2, 128))
    _, y = ora.rope(x, np.zeros(3, np.int32), rp)
    xd = ora.f16_to_f64(x)
    np.testing.assert_allclose(y[..., 64:], xd[..., 64:] * rp.mscale, rtol=1e-15)
    assert np.array_equal(y[..., :64], xd[..., :64])


# ---------------------------------------------------------------- rotation variants
# Half-split pairing (pair j = dims (o + j, o + j + n_rot/2)), the inverse rotation
# (ds4 Trace 2's `inverse` flag: the sine's sign flipped) and caller tables of cos / sin
# gathered by position (Sophgo Listings 1-2: top.Gather(rotary_cos_w, pos_ids)).

def _interleave(x, n_rot):
    """Dims o + j and o + j + n_rot/2 of x placed at o + 2j and o + 2j + 1."""
    d = x.shape[-1]
    o, half = d - n_rot, n_rot // 2
    y = x.copy()
    y[..., o + 0:d:2] = x[..., o:o + half]
    y[..., o + 1:d:2] = x[..., o + half:d]
    return y


@pytest.mark.parametrize("rp_name", ["plain", "yarn"])
def test_half_split_is_adjacent_rotation_of_permuted_dims(ora, rp_name):
    # The same rotation on a permuted pairing: interleaving the two halves, rotating with
    # adjacent pairs and de-interleaving gives the half-split result bit for bit.
    rp = ora.RopeParams.plain() if rp_name == "plain" else ora.RopeParams.yarn_tail()
    rng = np.random.default_rng(21)
    x = _rand_f16(rng, (9, 2, 128))
    pos = rng.integers(0, 30000, 9).astype(np.int32)
    hs, hs64 = ora.rope(x, pos, rp.replace(half_split=True))
    adj, adj64 = ora.rope(_interleave(x, rp.n_rot), pos, rp)
    assert np.array_equal(_interleave(hs, rp.n_rot), adj)
    assert np.array_equal(_interleave(hs64, rp.n_rot), adj64)
    # and it is a different pairing (dims really move between pairs)
    assert not np.array_equal(hs, ora.rope(x, pos, rp)[0])


def test_half_split_matches_complex_multiplication(ora):
    # independent route: (x[j] + i x[j + 64]) * exp(i pos base^(-2j/128)) in complex128
    rng = np.random.default_rng(22)
    rows = 24
    x = _rand_f16(rng, (rows, 2, 128))
    pos = rng.integers(0, 5000, rows).astype(np.int32)
    _, y = ora.rope(x, pos, ora.RopeParams.plain().replace(half_split=True))
    xd = x.view(np.float16).astype(np.float64)
    z = xd[..., :64] + 1j * xd[..., 64:]
    freqs = np.power(10000.0, -np.arange(64) / 64.0)
    w = z * np.exp(1j * pos[:, None, None] * freqs[None, None, :])
    np.testing.assert_allclose(y[..., :64], w.real, atol=1e-11)
    np.testing.assert_allclose(y[..., 64:], w.imag, atol=1e-11)


def test_half_split_tail_keeps_head_dims(ora):
    rp = ora.RopeParams.yarn_tail().replace(half_split=True)
    rng = np.random.default_rng(23)
    x = _rand_f16(rng, (6, 4, 128))
    out, _ = ora.rope(x, rng.integers(1, 9000, 6).astype(np.int32), rp)
    assert np.array_equal(out[..., :64], x[..., :64])
    assert not np.array_equal(out[..., 64:], x[..., 64:])


@pytest.mark.parametrize("rp_name", ["plain", "yarn", "half"])
def test_inverse_at_pos_is_forward_at_minus_pos(ora, rp_name):
    # R(-theta) = R(theta)^T: the inverse at p equals the forward rotation at -p, bit for
    # bit (cos is even and sin odd, exactly, in fp64).
    rp = {"plain": ora.RopeParams.plain(), "yarn": ora.RopeParams.yarn_tail(),
          "half": ora.RopeParams.plain().replace(half_split=True)}[rp_name]
    rng = np.random.default_rng(24)
    x = _rand_f16(rng, (11, 2, 128))
    pos = rng.integers(0, 20000, 11).astype(np.int32)
    inv, inv64 = ora.rope(x, pos, rp.replace(inverse=True))
    fwd, fwd64 = ora.rope(x, -pos, rp)
    assert np.array_equal(inv, fwd)
    assert np.array_equal(inv64, fwd64)


def test_inverse_undoes_forward_in_fp64(ora):
    # closed form: the inverse rotation of the exact forward rotation returns x; checked
    # in complex128 as z * exp(i t) * exp(-i t) with the oracle supplying both halves
    rng = np.random.default_rng(25)
    x = _rand_f16(rng, (8, 1, 128))
    pos = rng.integers(0, 4000, 8).astype(np.int32)
    _, y = ora.rope(x, pos, ora.RopeParams.plain().replace(inverse=True))
    xd = x.view(np.float16).astype(np.float64)
    z = xd[..., 0::2] + 1j * xd[..., 1::2]
    freqs = np.power(10000.0, -np.arange(64) / 64.0)
    w = z * np.exp(-1j * pos[:, None, None] * freqs[None, None, :])
    np.testing.assert_allclose(y[..., 0::2], w.real, atol=1e-11)
    np.testing.assert_allclose(y[..., 1::2], w.imag, atol=1e-11)


def _tables(rows, n_rot, base=10000.0):
    j = np.arange(n_rot // 2)
    ang = np.arange(rows)[:, None] * np.power(base, -2.0 * j / n_rot)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@pytest.mark.parametrize("half_split", [False, True])
def test_table_rotation_closed_form(ora, half_split):
    # with tables, each pair turns by the gathered (cos, sin): checked in complex128
    # against the float32 table values themselves
    rng = np.random.default_rng(26)
    ct, st = _tables(3000, 128)
    x = _rand_f16(rng, (10, 3, 128))
    pos = rng.integers(0, 3000, 10).astype(np.int32)
    rp = ora.RopeParams.plain().replace(cos_table=ct, sin_table=st, half_split=half_split)
    _, y = ora.rope(x, pos, rp)
    xd = x.view(np.float16).astype(np.float64)
    a, b = (xd[..., :64], xd[..., 64:]) if half_split else (xd[..., 0::2], xd[..., 1::2])
    rot = ct[pos].astype(np.float64)[:, None, :] + 1j * st[pos].astype(np.float64)[:, None, :]
    w = (a + 1j * b) * rot
    ya, yb = (y[..., :64], y[..., 64:]) if half_split else (y[..., 0::2], y[..., 1::2])
    np.testing.assert_allclose(ya, w.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(yb, w.imag, rtol=0, atol=1e-12)


def test_table_gather_follows_positions(ora):
    # identity rows rotate nothing; permuting the table rows together with the positions
    # changes nothing; a position past the table makes the rotated dims NaN
    rng = np.random.default_rng(27)
    ct, st = _tables(64, 64)
    x = _rand_f16(rng, (6, 2, 128))
    pos = np.array([0, 5, 63, 17, 40, 2], np.int32)
    rp = ora.RopeParams.yarn_tail().replace(cos_table=ct, sin_table=st)
    out, _ = ora.rope(x, pos, rp)
    perm = rng.permutation(64)
    inv = np.argsort(perm)
    out_p, _ = ora.rope(x, inv[pos].astype(np.int32), rp.replace(cos_table=ct[perm], sin_table=st[perm]))
    assert np.array_equal(out, out_p)
    one, zero = np.ones_like(ct), np.zeros_like(st)
    ident, _ = ora.rope(x, pos, rp.replace(cos_table=one, sin_table=zero))
    assert np.array_equal(ident, x)
    bad, bad64 = ora.rope(x, np.array([0, 64, -1, 3, 3, 3], np.int32), rp)
    assert np.isnan(bad64[1:3, :, 64:]).all() and not np.isnan(bad64[[0, 3], :, 64:]).any()
    assert np.array_equal(bad[1:3, :, :64], x[1:3, :, :64])


def test_table_of_the_schedule_matches_computed_rotation(ora):
    # tables holding fp32-rounded cos / sin of the plain schedule agree with the computed
    # rotation to fp32 accuracy of the factors
    rng = np.random.default_rng(28)
    ct, st = _tables(5000, 128)
    x = _rand_f16(rng, (12, 2, 128))
    pos = rng.integers(0, 5000, 12).astype(np.int32)
    _, yt = ora.rope(x, pos, ora.RopeParams.plain().replace(cos_table=ct, sin_table=st))
    _, yc = ora.rope(x, pos, ora.RopeParams.plain())
    np.testing.assert_allclose(yt, yc, rtol=0, atol=5e-7 * np.abs(x.view(np.float16)).max() * 2)
