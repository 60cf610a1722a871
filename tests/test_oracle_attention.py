"""Pins for the oracle's causal grouped-query attention and the three phases.

What the pages fix:
  * FAttention = scaled dot product + causal mask (Sophgo paper, sec. 2.2);
  * prefill_kv concatenates the history before the new tokens (Listing 2, sec. 4.1),
    decode is one query over every earlier key (sec. 4.1);
  * query head h reads KV head floor(h / G) (CGDR notes, sec. 1-2: repeat_interleave);
  * the decode position is the current cache length, +1 per step (Buddy-MLIR
    walkthrough, sec. 6.4.5-6.4.6).
The checks below use limiting cases with closed forms, an independent library route
(torch float64 scaled_dot_product_attention with an explicit mask), and the consistency
of the oracle's two separately written attention loops.
"""
import numpy as np
import pytest
import torch


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float16).view(np.uint16)


def _case(rng, n, t, hq, hkv, d, lens, s_cap):
    q = _rand(rng, (n, t, hq, d))
    k = _rand(rng, (n, t, hkv, d))
    v = _rand(rng, (n, t, hkv, d))
    ck = np.zeros((n, hkv, s_cap, d), np.uint16)
    cv = np.zeros_like(ck)
    for u in range(n):
        ck[u, :, : lens[u]] = _rand(rng, (hkv, lens[u], d))
        cv[u, :, : lens[u]] = _rand(rng, (hkv, lens[u], d))
    pos = (np.asarray(lens)[:, None] + np.arange(t)[None, :]).astype(np.int32)
    return q, k, v, pos, ck, cv


def _f64(ora, a):
    return ora.f16_to_f64(a)


def test_single_token_returns_its_value_row(ora):
    rng = np.random.default_rng(10)
    q, k, v, pos, ck, cv = _case(rng, 3, 1, 6, 2, 128, [0, 0, 0], 4)
    out, out64, _ = ora.prefill(q, k, v, pos, ck, cv, 0.0883883, ora.RopeParams.plain())
    G = 3
    for h in range(6):
        assert np.array_equal(out[:, 0, h], v[:, 0, h // G])


def test_zero_query_gives_prefix_mean(ora):
    rng = np.random.default_rng(11)
    n, t, hq, hkv, d = 2, 9, 4, 2, 16
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, [0, 0], 9)
    q[:] = 0
    _, out64, _ = ora.prefill(q, k, v, pos, ck, cv, 0.25, ora.RopeParams.plain(n_rot=16))
    vd = _f64(ora, v)
    for u in range(n):
        for h in range(hq):
            for tt in range(t):
                ref = vd[u, : tt + 1, h // 2].mean(axis=0)
                np.testing.assert_allclose(out64[u, tt, h], ref, rtol=1e-14, atol=1e-15)


def test_probabilities_sum_to_one(ora):
    # with every value row equal to 1 the output is the sum of the probabilities
    rng = np.random.default_rng(12)
    n, t, hq, hkv, d = 2, 13, 6, 2, 128
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, [5, 0], 20)
    one = np.float16(1.0).view(np.uint16)
    v[:] = one
    cv[:, :, :5] = one
    _, out64, _ = ora.prefill_kv(q, k, v, pos, ck, cv, [5, 0], 0.0883883,
                                 ora.RopeParams.plain())
    np.testing.assert_allclose(out64, 1.0, rtol=0, atol=1e-14)


def test_planted_maximum_selects_its_row(ora):
    # a huge scale turns softmax into argmax: with the query equal to key row 2 (and
    # much larger than the others), every query that can see row 2 returns V row 2.
    n, t, hq, hkv, d = 1, 6, 2, 1, 8
    q = np.zeros((n, t, hq, d), np.float16)
    k = np.full((n, t, hkv, d), 0.01, np.float16)
    v = np.arange(n * t * hkv * d, dtype=np.float16).reshape(n, t, hkv, d) / 8
    k[0, 2, 0, :] = 3.0
    q[0, :, :, :] = 3.0
    pos = np.zeros((n, t), np.int32)   # position 0 everywhere: no rotation
    ck = np.zeros((n, hkv, t, d), np.uint16)
    cv = np.zeros_like(ck)
    out, _, _ = ora.prefill(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), pos,
                            ck, cv, 1e3, ora.RopeParams.plain(n_rot=8))
    for tt in range(2, t):
        assert np.array_equal(out[0, tt, 0], v.view(np.uint16)[0, 2, 0])


def _torch_reference(ora, q, k, v, pos, ck, cv, lens, scale, rp):
    """Independent route: RoPE by complex multiplication (numpy), f16 rounding by numpy,
    attention by torch float64 SDPA with an explicit boolean mask over the
    concatenation [history; new] and repeat_interleave for the KV heads."""
    n, t, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    o = d - rp.n_rot
    freqs = np.power(rp.base, -np.arange(rp.n_rot // 2) / (rp.n_rot / 2))

    def rot(x16):
        x = x16.view(np.float16).astype(np.float64)
        z = x[..., o::2] + 1j * x[..., o + 1::2]
        z = z * np.exp(1j * pos[:, :, None, None] * freqs)
        y = x.copy()
        y[..., o::2], y[..., o + 1::2] = z.real, z.imag
        return y.astype(np.float16).astype(np.float64)

    qr, kr = rot(q), rot(k)
    vd = v.view(np.float16).astype(np.float64)
    outs = np.zeros((n, t, hq, d))
    for u in range(n):
        L = lens[u] + t
        hk = ck[u, :, : lens[u]].view(np.float16).astype(np.float64)
        hv = cv[u, :, : lens[u]].view(np.float16).astype(np.float64)
        K = np.concatenate([hk, kr[u].transpose(1, 0, 2)], axis=1)   # [hkv, L, d]
        V = np.concatenate([hv, vd[u].transpose(1, 0, 2)], axis=1)
        Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)          # [hq, L, d]
        Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
        Qt = torch.from_numpy(qr[u].transpose(1, 0, 2).copy())         # [hq, t, d]
        mask = torch.arange(L)[None, :] <= (lens[u] + torch.arange(t))[:, None]
        res = torch.nn.functional.scaled_dot_product_attention(
            Qt, Kt, Vt, attn_mask=mask, scale=scale)
        outs[u] = res.numpy().transpose(1, 0, 2)
    return outs


@pytest.mark.parametrize("t,hq,hkv,d,lens", [
    (17, 6, 6, 8, [0, 3]),      # G = 1 (MHA)
    (5, 4, 2, 128, [0, 9]),     # G = 2
    (11, 6, 2, 8, [4, 0]),      # G = 3
    (16, 12, 2, 128, [0, 1]),   # G = 6
    (1, 6, 1, 128, [7, 0]),     # single token, G = 6
])
def test_brute_force_torch_float64(ora, t, hq, hkv, d, lens):
    rng = np.random.default_rng(20 + t + d)
    n = len(lens)
    s_cap = max(lens) + t + 2
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, lens, s_cap)
    rp = ora.RopeParams.plain(n_rot=d)
    ref = _torch_reference(ora, q, k, v, pos, ck.copy(), cv.copy(), lens, 0.3, rp)
    _, out64, _ = ora.prefill_kv(q, k, v, pos, ck, cv, lens, 0.3, rp)
    np.testing.assert_allclose(out64, ref, rtol=1e-10, atol=1e-12)


def test_prefill_equals_successive_decodes(ora):
    rng = np.random.default_rng(30)
    n, t, hq, hkv, d = 2, 12, 6, 2, 128
    for rp in [ora.RopeParams.plain(), ora.RopeParams.yarn_tail()]:
        q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, [0, 0], t)
        ck2, cv2 = ck.copy(), cv.copy()
        out, out64, _ = ora.prefill(q, k, v, pos, ck, cv, 0.0883883, rp)
        for tt in range(t):
            o2, o2_64, _ = ora.decode(q[:, tt].copy(), k[:, tt].copy(), v[:, tt].copy(),
                                      pos[:, tt].copy(), ck2, cv2,
                                      np.full(n, tt, np.int32), 0.0883883, rp)
            np.testing.assert_allclose(o2_64, out64[:, tt], rtol=1e-12, atol=1e-13)
            assert np.array_equal(o2, out[:, tt])
        assert np.array_equal(ck, ck2) and np.array_equal(cv, cv2)


def test_prefill_kv_equals_tail_of_full_prefill(ora):
    rng = np.random.default_rng(31)
    n, t, hq, hkv, d, hist = 2, 20, 4, 2, 128, 13
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, [0, 0], t)
    out, out64, _ = ora.prefill(q, k, v, pos, ck, cv, 0.1, ora.RopeParams.plain())
    # history = first `hist` rows of the full prefill's cache; new = the rest
    hk = np.zeros_like(ck)
    hv = np.zeros_like(cv)
    hk[:, :, :hist] = ck[:, :, :hist]
    hv[:, :, :hist] = cv[:, :, :hist]
    out2, out2_64, _ = ora.prefill_kv(q[:, hist:].copy(), k[:, hist:].copy(),
                                      v[:, hist:].copy(), pos[:, hist:].copy(), hk, hv,
                                      np.full(n, hist, np.int32), 0.1, ora.RopeParams.plain())
    np.testing.assert_allclose(out2_64, out64[:, hist:], rtol=1e-12, atol=1e-13)
    assert np.array_equal(out2, out[:, hist:])
    assert np.array_equal(hk, ck) and np.array_equal(hv, cv)


def test_group_sharing_equals_duplicated_kv_heads(ora):
    rng = np.random.default_rng(32)
    n, t, hq, hkv, d = 1, 7, 6, 2, 128
    G = hq // hkv
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, [3], 12)
    out, _, _ = ora.prefill_kv(q, k, v, pos, ck.copy(), cv.copy(), [3], 0.09,
                               ora.RopeParams.plain())
    k6 = np.repeat(k, G, axis=2)
    v6 = np.repeat(v, G, axis=2)
    ck6 = np.repeat(ck, G, axis=1)
    cv6 = np.repeat(cv, G, axis=1)
    out6, _, _ = ora.prefill_kv(q, k6, v6, pos, ck6, cv6, [3], 0.09, ora.RopeParams.plain())
    assert np.array_equal(out, out6)


def test_append_writes_only_its_rows(ora):
    rng = np.random.default_rng(33)
    n, t, hkv, d, s_cap = 3, 4, 2, 16, 12
    ck = _rand(rng, (n, hkv, s_cap, d))
    cv = _rand(rng, (n, hkv, s_cap, d))
    k = _rand(rng, (n, t, hkv, d))
    v = _rand(rng, (n, t, hkv, d))
    lens = np.array([0, 5, 8], np.int32)
    ck0, cv0 = ck.copy(), cv.copy()
    ora.append(ck, cv, k, v, lens)
    for u in range(n):
        rows = np.arange(s_cap)
        new = (rows >= lens[u]) & (rows < lens[u] + t)
        assert np.array_equal(ck[u][:, ~new], ck0[u][:, ~new])
        assert np.array_equal(cv[u][:, ~new], cv0[u][:, ~new])
        assert np.array_equal(ck[u][:, new], k[u].transpose(1, 0, 2))
        assert np.array_equal(cv[u][:, new], v[u].transpose(1, 0, 2))
    with pytest.raises(ValueError):
        ora.append(ck, cv, k, v, np.array([0, 5, 9], np.int32))


def test_capacity_error_is_raised(ora):
    rng = np.random.default_rng(35)
    q, k, v, pos, ck, cv = _case(rng, 1, 4, 2, 1, 8, [0], 4)
    with pytest.raises(ValueError):
        ora.prefill_kv(q, k, v, pos, ck, cv, [1], 0.3, ora.RopeParams.plain(n_rot=8))
    with pytest.raises(ValueError):
        ora.decode(q[:, 0].copy(), k[:, 0].copy(), v[:, 0].copy(), pos[:, 0].copy(), ck, cv,
                   [4], 0.3, ora.RopeParams.plain(n_rot=8))


def test_varlen_with_full_counts_equals_batched_prefill_kv(ora):
    rng = np.random.default_rng(36)
    n, t, hq, hkv, d = 3, 9, 6, 2, 128
    lens = [0, 5, 11]
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, lens, 24)
    ck2, cv2 = ck.copy(), cv.copy()
    out, out64, k64 = ora.prefill_kv(q, k, v, pos, ck, cv, lens, 0.09, ora.RopeParams.plain())
    o2, o2_64, k2 = ora.prefill_kv_varlen(q, k, v, pos, ck2, cv2, lens, [t] * n, 0.09,
                                          ora.RopeParams.plain())
    assert np.array_equal(out, o2) and np.array_equal(out64, o2_64) and np.array_equal(k64, k2)
    assert np.array_equal(ck, ck2) and np.array_equal(cv, cv2)


def test_varlen_units_equal_their_own_successive_decodes(ora):
    # each unit's valid rows against the decode loop (a separately written attention loop),
    # one step per new token; padding rows hold NaN and change nothing; cache rows past each
    # unit's new tokens stay as they were
    rng = np.random.default_rng(37)
    n, t, hq, hkv, d = 4, 8, 4, 2, 128
    lens, new = [0, 6, 3, 9], [8, 1, 0, 5]
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, lens, 20)
    nan16 = np.uint16(0x7e00)
    for u in range(n):
        q[u, new[u]:] = nan16
        k[u, new[u]:] = nan16
        v[u, new[u]:] = nan16
    ck0, cv0 = ck.copy(), cv.copy()
    rp = ora.RopeParams.yarn_tail()
    out, out64, _ = ora.prefill_kv_varlen(q, k, v, pos, ck, cv, lens, new, 0.09, rp)
    for u in range(n):
        cku, cvu = ck0[u:u + 1].copy(), cv0[u:u + 1].copy()
        for i in range(new[u]):
            o, o64, _ = ora.decode(q[u:u + 1, i].copy(), k[u:u + 1, i].copy(), v[u:u + 1, i].copy(),
                                   pos[u:u + 1, i].copy(), cku, cvu, np.array([lens[u] + i], np.int32),
                                   0.09, rp)
            np.testing.assert_allclose(out64[u, i], o64[0], rtol=1e-12, atol=1e-13)
        assert np.array_equal(ck[u], cku[0]) and np.array_equal(cv[u], cvu[0])
        assert np.isnan(out64[u, new[u]:]).all()
        assert np.array_equal(ck[u][:, lens[u] + new[u]:], ck0[u][:, lens[u] + new[u]:])
    assert np.all(np.isfinite(out64[0])) and np.all(np.isfinite(out64[1, :1]))


def test_unit_parameter_sets_equal_separate_calls(ora):
    # ds4.c study notes, Part 4 sec. 1, Trace 2: each layer has its own frequency base and
    # scale, and only the compressed layers switch the YaRN ramp on (ext_factor > 0).  A
    # batch whose units use different parameter sets computes, for every unit, exactly
    # what a call with that unit's set alone computes: outputs, rotated k and caches.
    rng = np.random.default_rng(38)
    n, t, hq, hkv, d = 4, 9, 8, 2, 128
    plain = ora.RopeParams.plain()
    compressed = ora.RopeParams(base=160000.0, n_rot=64, yarn=True, freq_scale=1.0 / 16,
                                ext_factor=1.0, n_ctx_orig=65536, beta_fast=32.0, beta_slow=1.0,
                                mscale=1.0 + 0.1 * np.log(16.0))
    sets, unit_set = [plain, compressed], np.array([1, 0, 0, 1], np.int32)
    lens = [0, 7, 30, 12]
    q, k, v, pos, ck, cv = _case(rng, n, t, hq, hkv, d, lens, 48)
    ck_b, cv_b = ck.copy(), cv.copy()
    out, out64, k64 = ora.prefill_kv(q, k, v, pos, ck_b, cv_b, lens, 0.09, sets, unit_set)
    for u in range(n):
        cku, cvu = ck[u:u + 1].copy(), cv[u:u + 1].copy()
        o, o64, kk = ora.prefill_kv(q[u:u + 1], k[u:u + 1], v[u:u + 1], pos[u:u + 1], cku, cvu,
                                    lens[u:u + 1], 0.09, sets[unit_set[u]])
        assert np.array_equal(o[0], out[u]) and np.array_equal(o64[0], out64[u])
        assert np.array_equal(kk[0], k64[u]) and np.array_equal(cku[0], ck_b[u])
        assert np.array_equal(cvu[0], cv_b[u])
    # the two sets really differ on these inputs
    o_plain, _, _ = ora.prefill_kv(q, k, v, pos, ck.copy(), cv.copy(), lens, 0.09, plain)
    assert not np.array_equal(o_plain[0], out[0]) and np.array_equal(o_plain[1], out[1])
    # decode: the same, one step
    qd, kd, vd = q[:, 0].copy(), k[:, 0].copy(), v[:, 0].copy()
    dl = np.array(lens, np.int32) + 3
    ck_b, cv_b = ck.copy(), cv.copy()
    out, out64, _ = ora.decode(qd, kd, vd, dl, ck_b, cv_b, dl, 0.09, sets, unit_set)
    for u in range(n):
        cku, cvu = ck[u:u + 1].copy(), cv[u:u + 1].copy()
        o, o64, _ = ora.decode(qd[u:u + 1], kd[u:u + 1], vd[u:u + 1], dl[u:u + 1], cku, cvu, dl[u:u + 1],
                               0.09, sets[unit_set[u]])
        assert np.array_equal(o64[0], out64[u]) and np.array_equal(cku[0], ck_b[u])
