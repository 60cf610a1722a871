"""GPU parity of the projections either side of attention (fused QKV projection with k
rotation and cache append; output projection with the residual) against the CPU oracle,
and of the whole block (projection -> attention over the appended caches -> output
projection).

Bars, written here:
  * a projected value (q, v, out) is the f16 rounding of an fp32-accumulated dot product:
    within half an f16 ulp of the oracle's exact fp64 value plus the fp32 accumulation
    bound K * 2^-24 * sum_i |a_i w_i| (a rounding boundary can fall between the two);
  * a rotated k row element is the fp64 rotation of a projected k that may sit one ulp away
    from the oracle's: within 2 f16 ulps (at the norm of its rotation pair) plus twice the
    fp32 accumulation bound (times mscale) of the oracle's rotated k, and identical for the
    overwhelming majority (checked: at most 2 % differ);
  * untouched cache rows bit-identical;
  * the whole block: within 1e-2 absolute of the oracle's block output (the attention's
    2e-3 bar carried through the output projection, plus its own rounding).
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_causal_rope_amd import workloads as W
from tests import parity as P
from tests.test_gpu_parity import bits, kv, ora_rope  # noqa: F401

pytestmark = pytest.mark.gpu


def ulp16(x):
    return np.spacing(np.abs(x).astype(np.float16)).astype(np.float64)


def check_projected(got_bits, ref64, acc_bound, what):
    g = got_bits.view(np.float16).astype(np.float64)
    err = np.abs(g - ref64)
    lim = 0.5 * ulp16(ref64) + acc_bound + 1e-12
    bad = err > lim
    assert not bad.any(), f"{what}: {int(bad.sum())} values off by more than half an ulp + fp32 bound " \
                          f"(worst {float((err - lim).max()):.3e})"


def acc_bound(a_bits, w_bits, k):
    """K 2^-24 sum |a_i w_i| for every output (the fp32 accumulation bound)."""
    a = np.abs(a_bits.view(np.float16).astype(np.float64))
    w = np.abs(w_bits.view(np.float16).astype(np.float64))
    return k * 2.0 ** -24 * (a @ w.T)


def pair_norm(r, n_rot, half_split):
    """Per element: the norm of its rotation pair (rotated dims) or |value| (the others)."""
    d = r.shape[-1]
    o = d - n_rot
    out = np.abs(r).copy()
    if half_split:
        a, b = r[..., o:o + n_rot // 2], r[..., o + n_rot // 2:]
        m = np.sqrt(a * a + b * b)
        out[..., o:o + n_rot // 2] = m
        out[..., o + n_rot // 2:] = m
    else:
        a, b = r[..., o::2], r[..., o + 1::2]
        m = np.sqrt(a * a + b * b)
        out[..., o::2] = m
        out[..., o + 1::2] = m
    return out


def make(g, shape, scale=1.0):
    return (torch.randn(shape, generator=g) * scale).half()


@pytest.mark.parametrize("n,t,hidden,hq,hkv,lens,rope,per_unit,half", [
    (2, 200, 256, 4, 2, [0, 37], W.PLAIN_128, False, False),
    (3, 64, 1536, 12, 2, [5, 0, 100], W.PLAIN_128, True, False),
    (1, 130, 512, 8, 8, [300], W.YARN_TAIL_64, False, True),
])
def test_qkv_project(kv, n, t, hidden, hq, hkv, lens, rope, per_unit, half):
    g = torch.Generator().manual_seed(60 + t)
    d = 128
    rows = (hq + 2 * hkv) * d
    x = make(g, (n, t, hidden))
    w = make(g, (n, rows, hidden) if per_unit else (rows, hidden), hidden ** -0.5)
    s_cap = max(lens) + t + 3
    ck = make(g, (n, hkv, s_cap, d))
    cv = make(g, (n, hkv, s_cap, d))
    pos = (torch.tensor(lens, dtype=torch.int32)[:, None] + torch.arange(t, dtype=torch.int32)[None, :]).contiguous()
    lens_t = torch.tensor(lens, dtype=torch.int32)
    orp = ora_rope(rope).replace(half_split=half)
    # oracle: exact projection rounded to f16, rotation of k, append
    qr, kr, vr = oracle.qkv_project(bits(x), bits(w), hq, hkv)
    rk, rv = bits(ck).copy(), bits(cv).copy()
    k_rot, k64 = oracle.rope(kr.reshape(n * t, hkv, d), pos.numpy().reshape(-1), orp)
    oracle.append(rk, rv, k_rot.reshape(n, t, hkv, d), vr, lens)
    # GPU
    ckd, cvd = ck.cuda(), cv.cuda()
    lib = kv.RopeParams.from_fields(rope).with_variant(half_split=half)
    q = kv.qkv_project(x.cuda(), w.cuda(), pos.cuda(), ckd, cvd, lens_t.cuda(), max(lens), lib, hq, hkv)
    torch.cuda.synchronize()
    # q and v against the exact projection
    xb, wb = bits(x), bits(w)
    for u in range(n):
        wu = wb[u] if per_unit else wb
        y64, _ = oracle.project(xb[u], wu)
        bound = acc_bound(xb[u], wu, hidden)
        check_projected(bits(q)[u].reshape(t, hq * d), y64[:, : hq * d], bound[:, : hq * d], f"q unit {u}")
        gv = bits(cvd)[u][:, lens[u]:lens[u] + t]                       # [hkv, t, d]
        vref = y64[:, (hq + hkv) * d:].reshape(t, hkv, d).transpose(1, 0, 2)
        vbound = bound[:, (hq + hkv) * d:].reshape(t, hkv, d).transpose(1, 0, 2)
        check_projected(gv, vref, vbound, f"v unit {u}")
    # cache rows: untouched ones bit-identical, K rows within 2 ulps of the oracle's rotation
    gk = bits(ckd)
    k_differ = 0
    for u in range(n):
        wu = wb[u] if per_unit else wb
        # fp32 accumulation bound of each projected k value, [hkv, t, d]; a rotation mixes
        # two of them (times mscale)
        kb = acc_bound(xb[u], wu, hidden)[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d).transpose(1, 0, 2)
        kb = 2 * rope.mscale * kb.max(axis=-1, keepdims=True)
        new = slice(lens[u], lens[u] + t)
        untouched = np.ones(s_cap, bool)
        untouched[new] = False
        assert np.array_equal(gk[u][:, untouched], rk[u][:, untouched]), "untouched K rows changed"
        assert np.array_equal(bits(cvd)[u][:, untouched], rv[u][:, untouched]), "untouched V rows changed"
        gf = gk[u][:, new].view(np.float16).astype(np.float64)
        rf = rk[u][:, new].view(np.float16).astype(np.float64)
        # a one-ulp change of a projected k moves a rotated value by up to an ulp of its
        # pair's norm: the bound is two ulps at that norm
        lim = 2 * ulp16(pair_norm(rf, rope.n_rot, half)) + kb + 1e-12
        assert np.all(np.abs(gf - rf) <= lim), f"unit {u}: rotated K beyond 2 ulps of the pair norm"
        k_differ += int((gk[u][:, new] != rk[u][:, new]).sum())
    assert k_differ <= 0.02 * n * hkv * t * d, f"{k_differ} rotated K values differ from the oracle's"


@pytest.mark.parametrize("n,t,hq,hidden,per_unit", [(2, 150, 4, 256, False), (3, 64, 12, 1536, True)])
def test_out_project(kv, n, t, hq, hidden, per_unit):
    g = torch.Generator().manual_seed(70 + t)
    d = 128
    attn = make(g, (n, t, hq, d))
    w = make(g, (n, hidden, hq * d) if per_unit else (hidden, hq * d), (hq * d) ** -0.5)
    res = make(g, (n, t, hidden))
    y64, _ = oracle.out_project(bits(attn).reshape(n, t, hq * d), bits(w), bits(res))
    out = kv.out_project(attn.cuda(), w.cuda(), res.cuda())
    torch.cuda.synchronize()
    ab, wb = bits(attn).reshape(n, t, hq * d), bits(w)
    for u in range(n):
        bound = acc_bound(ab[u], wb[u] if per_unit else wb, hq * d)
        check_projected(bits(out)[u], y64[u], bound, f"out unit {u}")


def test_block_projection_attention_projection(kv):
    """x -> fused QKV projection (k rotated, k/v appended) -> attention over the caches ->
    output projection + residual, against the oracle's block on the same inputs."""
    g = torch.Generator().manual_seed(80)
    n, t, hidden, hq, hkv, d = 2, 96, 512, 8, 2, 128
    lens = [0, 40]
    s_cap = max(lens) + t + 1
    rope = W.PLAIN_128
    x = make(g, (n, t, hidden))
    w_qkv = make(g, ((hq + 2 * hkv) * d, hidden), hidden ** -0.5)
    w_o = make(g, (hidden, hq * d), (hq * d) ** -0.5)
    ck = make(g, (n, hkv, s_cap, d))
    cv = make(g, (n, hkv, s_cap, d))
    pos = (torch.tensor(lens, dtype=torch.int32)[:, None] + torch.arange(t, dtype=torch.int32)[None, :]).contiguous()
    scale = d ** -0.5
    # oracle block
    qr, kr, vr = oracle.qkv_project(bits(x), bits(w_qkv), hq, hkv)
    rk, rv = bits(ck).copy(), bits(cv).copy()
    att, _, _ = oracle.prefill_kv(qr, kr, vr, pos.numpy(), rk, rv, np.asarray(lens, np.int32), scale,
                                  ora_rope(rope))
    y64, _ = oracle.out_project(att.reshape(n, t, hq * d), bits(w_o), bits(x))
    # GPU block
    rp = kv.RopeParams.from_fields(rope)
    xd, ckd, cvd = x.cuda(), ck.cuda(), cv.cuda()
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = kv.qkv_project(xd, w_qkv.cuda(), pos.cuda(), ckd, cvd, lens_d, max(lens), rp, hq, hkv)
    o = kv.prefill_kv_cached(q, pos.cuda(), ckd, cvd, lens_d, max(lens), rp, scale=scale)
    y = kv.out_project(o, w_o.cuda(), xd)
    torch.cuda.synchronize()
    err = np.abs(bits(y).view(np.float16).astype(np.float64) - y64)
    assert float(err.max()) <= 1e-2, f"block output max abs error {float(err.max()):.3e}"
