"""GPU parity: every entry point of libkvrope against the CPU oracle on the same seeded
inputs, at sizes the oracle finishes in seconds that still span several tiles, ragged
tails and every query-head group size the kernels specialise for.

Bars (see tests/parity.py): outputs within 2e-3 absolute and 1e-2 row-relative of the
oracle's fp64 result; V rows and untouched cache rows bit-identical; rotated K rows equal
to the oracle's f16 rounding (boundary cases counted).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from kv_cache_causal_rope_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import kv_cache_causal_rope_amd as kv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kv.lib()
    return kv


def ora_rope(r: W.Rope) -> oracle.RopeParams:
    return oracle.RopeParams(base=r.base, n_rot=r.n_rot, yarn=r.yarn, freq_scale=r.freq_scale,
                             ext_factor=r.ext_factor, n_ctx_orig=r.n_ctx_orig,
                             beta_fast=r.beta_fast, beta_slow=r.beta_slow, mscale=r.mscale)


def custom(n, t, hq, hkv, s_cap, rope=W.PLAIN_128, seed=100):
    return W.Config("custom", "prefill_kv", n, 1, t, hq, hkv, 128, rope, 0, 0, s_cap, seed, "")


def to_dev(inp: W.Inputs) -> W.Inputs:
    return W.Inputs(*[x.cuda() for x in dataclasses.astuple(inp)])


def bits(x):
    return P.to_np_bits(x)


# ------------------------------------------------------------------ rotary embedding
@pytest.mark.parametrize("rope,h,maxpos", [(W.PLAIN_128, 12, 5000), (W.YARN_TAIL_64, 8, 40000),
                                           (W.Rope(n_rot=2), 3, 100),
                                           (W.Rope(n_rot=38, base=500000.0), 5, 70000)])
def test_rope_apply_matches_oracle(kv, rope, h, maxpos):
    g = torch.Generator().manual_seed(11)
    n, t = 3, 37
    x = torch.randn((n, t, h, 128), generator=g).half()
    pos = torch.randint(0, maxpos, (n, t), generator=g, dtype=torch.int32)
    ref_bits, ref64 = oracle.rope(bits(x).reshape(n * t, h, 128), bits_pos(pos), ora_rope(rope))
    xd = x.cuda()
    kv.rope_apply(xd, pos.cuda(), kv.RopeParams.from_fields(rope))
    torch.cuda.synchronize()
    got = bits(xd).reshape(n * t, h, 128)
    P.check_k_rows(got, ref_bits, ref64, "rope_apply")


def bits_pos(pos):
    return pos.numpy().reshape(-1).astype(np.int32)


def test_cache_append_bit_exact(kv):
    g = torch.Generator().manual_seed(12)
    n, t, hkv, s_cap = 3, 5, 2, 16
    ck = torch.randn((n, hkv, s_cap, 128), generator=g).half()
    cv = torch.randn((n, hkv, s_cap, 128), generator=g).half()
    k = torch.randn((n, t, hkv, 128), generator=g).half()
    v = torch.randn((n, t, hkv, 128), generator=g).half()
    lens = torch.tensor([0, 7, 11], dtype=torch.int32)
    rk, rv = bits(ck).copy(), bits(cv).copy()
    oracle.append(rk, rv, bits(k), bits(v), lens.numpy())
    ckd, cvd = ck.cuda(), cv.cuda()
    kv.cache_append(ckd, cvd, k.cuda(), v.cuda(), lens.cuda(), 11)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ckd), rk) and np.array_equal(bits(cvd), rv)


# ------------------------------------------------------------------ prefill / prefill_kv
def run_prefill_kv(kv, cfg, lens, rope, poison=False, seed=None, spike=None):
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32), poison_tail=poison, seed=seed)
    if spike is not None:
        # Dim 0 (left unrotated by a tail rotation) set to 1 in every q row and to 2048 in
        # the new K row `spike` of every unit: rows that see that key score it some 250 log2
        # units above anything else, far past the f16 (and fp32) range of 2^(score - max),
        # while every other score keeps its size.  Both values are exact in f16.
        inp.q[..., 0] = 1.0
        inp.k[:, spike, :, 0] = 2048.0
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    ref_out, ref64, k64 = oracle.prefill_kv(bits(inp.q), bits(inp.k), bits(inp.v),
                                            inp.positions.numpy(), rk, rv, inp.lens.numpy(),
                                            cfg.scale, ora_rope(rope))
    d = to_dev(inp)
    out = kv.prefill_kv(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens,
                        int(max(lens)), kv.RopeParams.from_fields(rope), scale=cfg.scale)
    torch.cuda.synchronize()
    return inp, d, out, (ref_out, ref64, k64, rk, rv)


def check_prefill(d, out, ref, lens, t, what):
    ref_out, ref64, k64, rk, rv = ref
    P.check_attention(bits(out), ref64, what)
    gk, gv = bits(d.cache_k), bits(d.cache_v)
    assert np.array_equal(gv, rv), f"{what}: V cache differs"
    # K: rows outside the appended range must be identical; appended rows by the K rule
    n = gk.shape[0]
    for u in range(n):
        new = slice(lens[u], lens[u] + t)
        untouched = np.ones(gk.shape[2], bool)
        untouched[new] = False
        assert np.array_equal(gk[u][:, untouched], rk[u][:, untouched]), \
            f"{what}: untouched K rows changed"
        P.check_k_rows(gk[u][:, new], rk[u][:, new], k64[u].transpose(1, 0, 2), what)


def test_prefill_tiny_workload(kv):
    cfg = W.CONFIGS["tiny_prefill_t64"]
    inp, d, out, ref = run_prefill_kv(kv, cfg, [0], cfg.rope)
    check_prefill(d, out, ref, [0], cfg.t, cfg.name)


@pytest.mark.parametrize("n,t,hq,hkv", [
    (3, 77, 12, 2),   # G = 6, ragged tail, several tiles
    (2, 33, 4, 4),    # G = 1
    (1, 65, 6, 2),    # G = 3
    (2, 50, 16, 2),   # G = 8
    (1, 40, 32, 2),   # G = 16: two head slices per workgroup group
    (2, 1, 12, 2),    # single token
    (1, 130, 8, 4),   # G = 2
    (2, 70, 8, 1),    # one KV head (G = 8): the append kernel's single-head path
    (1, 48, 8, 8),    # eight KV heads, G = 1
])
def test_prefill_shapes(kv, n, t, hq, hkv):
    cfg = custom(n, t, hq, hkv, t + 3, seed=200 + t)
    lens = [0] * n
    inp, d, out, ref = run_prefill_kv(kv, cfg, lens, W.PLAIN_128)
    check_prefill(d, out, ref, lens, t, f"prefill n{n} t{t} {hq}/{hkv}")


@pytest.mark.parametrize("n,t,hq,hkv,lens,rope", [
    (2, 45, 32, 2, [37, 100], W.PLAIN_128),
    (3, 64, 12, 2, [0, 64, 130], W.PLAIN_128),
    (2, 29, 32, 8, [300, 5], W.YARN_TAIL_64),
    (1, 96, 6, 6, [1000], W.PLAIN_128),
    # history >= t and 32 KV pairs: the pair-major unit order, over two rounds of the grid
    (16, 200, 32, 2, [250 + 13 * u for u in range(16)], W.PLAIN_128),
    # history shorter than t: the lock-step layout (two workgroups per compute unit)
    (3, 100, 32, 2, [0, 37, 90], W.PLAIN_128),
])
def test_prefill_kv_shapes(kv, n, t, hq, hkv, lens, rope):
    cfg = custom(n, t, hq, hkv, max(lens) + t + 5, rope=rope, seed=300 + t)
    inp, d, out, ref = run_prefill_kv(kv, cfg, lens, rope)
    check_prefill(d, out, ref, lens, t, f"prefill_kv n{n} t{t} {hq}/{hkv} {lens}")


@pytest.mark.parametrize("n,t,hq,hkv,lens,new,rope", [
    (4, 70, 12, 2, [0, 100, 50, 7], [70, 1, 0, 33], W.PLAIN_128),
    (3, 45, 32, 8, [300, 0, 37], [45, 17, 44], W.YARN_TAIL_64),
    (2, 130, 8, 4, [0, 64], [129, 65], W.PLAIN_128),
])
def test_prefill_kv_varlen(kv, n, t, hq, hkv, lens, new, rope):
    """Units with different new-token counts in one call: padding rows hold NaN in q, k, v
    and must change nothing; their out rows keep the caller's values."""
    cfg = custom(n, t, hq, hkv, max(lens) + t + 5, rope=rope, seed=350 + t)
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    for u in range(n):
        for x in (inp.q, inp.k, inp.v):
            x[u, new[u]:] = float("nan")
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    rk0 = rk.copy()
    ref_out, ref64, k64 = oracle.prefill_kv_varlen(bits(inp.q), bits(inp.k), bits(inp.v),
                                                   inp.positions.numpy(), rk, rv, inp.lens.numpy(),
                                                   np.asarray(new, np.int32), cfg.scale, ora_rope(rope))
    d = to_dev(inp)
    out = torch.full_like(d.q, 7.0)
    kv.prefill_kv_varlen(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens,
                         torch.tensor(new, dtype=torch.int32, device="cuda"), int(max(lens)),
                         kv.RopeParams.from_fields(rope), scale=cfg.scale, out=out)
    torch.cuda.synchronize()
    got = bits(out)
    seven = np.float16(7.0).view(np.uint16)
    gk, gv = bits(d.cache_k), bits(d.cache_v)
    assert np.array_equal(gv, rv), "varlen: V cache differs"
    for u in range(n):
        what = f"varlen n{n} t{t} {hq}/{hkv} unit {u} ({lens[u]} + {new[u]})"
        if new[u]:
            P.check_attention(got[u, :new[u]], ref64[u, :new[u]], what)
        assert np.all(got[u, new[u]:] == seven), f"{what}: padding rows of out were written"
        rows = slice(lens[u], lens[u] + new[u])
        untouched = np.ones(gk.shape[2], bool)
        untouched[rows] = False
        assert np.array_equal(gk[u][:, untouched], rk0[u][:, untouched]), f"{what}: K rows changed"
        P.check_k_rows(gk[u][:, rows], rk[u][:, rows], k64[u, :new[u]].transpose(1, 0, 2), what)


def score_rise_log2(inp, ref, lens, rope, scale, hq, hkv):
    """Largest rise, over all rows, of a visible score above the row's max over keys
    0..63 (log2 units), from the oracle's rotated q and keys."""
    k64, rk = ref[2], ref[3]
    n, t = inp.q.shape[0], inp.q.shape[1]
    _, q64 = oracle.rope(bits(inp.q).reshape(n * t, hq, -1), inp.positions.numpy().reshape(-1),
                         ora_rope(rope))
    q64 = q64.reshape(n, t, hq, -1)
    g_size = hq // hkv
    rise = -np.inf
    for u in range(n):
        L = int(lens[u])
        for h in range(hq):
            g = h // g_size
            keys = np.concatenate([rk[u, g, :L].view(np.float16).astype(np.float64), k64[u][:, g, :]])
            sc = q64[u, :, h, :] @ keys.T * scale * np.log2(np.e)          # [t, L + t]
            for i in range(t):
                vis = sc[i, :L + i + 1]
                rise = max(rise, vis.max() - vis[:64].max())
    return rise


@pytest.mark.parametrize("n,t,hq,hkv,lens,spike", [
    (2, 130, 12, 2, [0, 0], 100),      # prefill
    (2, 45, 32, 2, [37, 100], 40),     # prefill_kv
])
def test_prefill_score_spike(kv, n, t, hq, hkv, lens, spike):
    rope = W.YARN_TAIL_64
    cfg = custom(n, t, hq, hkv, max(lens) + t + 5, rope=rope, seed=500 + t)
    inp, d, out, ref = run_prefill_kv(kv, cfg, lens, rope, spike=spike)
    # the spike does what it is meant to: some row's scores rise more than 16 (log2 units,
    # with the kernel's scale) above the max over its first 64 keys, so 2^(score - max)
    # leaves the f16 range and the kernel must fall back to its exact path
    assert score_rise_log2(inp, ref, lens, rope, cfg.scale, hq, hkv) > 16.0
    check_prefill(d, out, ref, lens, t, f"score-spike prefill n{n} t{t} {hq}/{hkv} {lens}")


@pytest.mark.parametrize("t", [50, 90])  # history 70 >= t: ping-pong layout; < t: lock-step
def test_prefill_poisoned_tail_is_never_read(kv, t):
    cfg = custom(2, t, 12, 2, 200, seed=400 + t)
    lens = [30, 70]
    inp, d, out, ref = run_prefill_kv(kv, cfg, lens, W.PLAIN_128, poison=True)
    check_prefill(d, out, ref, lens, t, f"prefill_kv t{t} poisoned")


# ------------------------------------------------------------------ decode
def run_decode(kv, n, hq, hkv, lens, s_cap, rope, seed, poison=False):
    cfg = W.Config("custom", "decode", n, 1, 1, hq, hkv, 128, rope, 0, 0, s_cap, seed, "")
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32), poison_tail=poison)
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    ref_out, ref64, k64 = oracle.decode(bits(inp.q)[:, 0], bits(inp.k)[:, 0], bits(inp.v)[:, 0],
                                        inp.positions.numpy()[:, 0], rk, rv, inp.lens.numpy(),
                                        cfg.scale, ora_rope(rope))
    d = to_dev(inp)
    out = kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, int(max(lens)),
                    kv.RopeParams.from_fields(rope), scale=cfg.scale)
    torch.cuda.synchronize()
    return d, out, (ref_out, ref64, k64, rk, rv)


def check_decode(d, out, ref, lens, what):
    ref_out, ref64, k64, rk, rv = ref
    P.check_attention(bits(out)[:, 0], ref64, what)
    gk, gv = bits(d.cache_k), bits(d.cache_v)
    assert np.array_equal(gv, rv), f"{what}: V cache differs"
    for u in range(gk.shape[0]):
        row = lens[u]
        P.check_k_rows(gk[u][:, row], rk[u][:, row], k64[u], what)
        others = np.ones(gk.shape[2], bool)
        others[row] = False
        assert np.array_equal(gk[u][:, others], rk[u][:, others]), f"{what}: K rows changed"


@pytest.mark.parametrize("n,hq,hkv,lens,rope", [
    (5, 12, 2, [0, 1, 63, 300, 129], W.PLAIN_128),      # G = 6
    (4, 32, 8, [700, 31, 512, 1], W.YARN_TAIL_64),       # G = 4, YaRN tail
    (3, 4, 4, [257, 2, 90], W.PLAIN_128),                # G = 1
    (2, 32, 2, [1500, 333], W.PLAIN_128),                # G = 16: two head slices
    (2, 6, 2, [4500, 2049], W.PLAIN_128),                # G = 3, multi-chunk
    (3, 16, 8, [255, 256, 257], W.PLAIN_128),            # G = 2, chunk boundaries (256-key minimum)
    (3, 10, 2, [40, 1700, 3], W.PLAIN_128),              # G = 5
    (2, 14, 2, [900, 77], W.YARN_TAIL_64),               # G = 7
    (3, 8, 1, [600, 5, 1300], W.PLAIN_128),              # one KV head, G = 8
])
def test_decode_shapes(kv, n, hq, hkv, lens, rope):
    d, out, ref = run_decode(kv, n, hq, hkv, lens, max(lens) + 3, rope, seed=500 + n)
    check_decode(d, out, ref, lens, f"decode {hq}/{hkv} {lens}")


def test_decode_poisoned_tail_is_never_read(kv):
    lens = [10, 200, 77]
    d, out, ref = run_decode(kv, 3, 12, 2, lens, 400, W.PLAIN_128, seed=600, poison=True)
    check_decode(d, out, ref, lens, "decode poisoned")


# ------------------------------------------------------------------ phase consistency
def test_gpu_prefill_equals_successive_gpu_decodes(kv):
    """Prefill of T tokens and T decode steps from an empty cache agree (GPU only)."""
    n, t, hq, hkv = 2, 40, 12, 2
    cfg = custom(n, t, hq, hkv, t, seed=700)
    inp = W.make_inputs(cfg, lens=np.zeros(n, np.int32))
    d = to_dev(inp)
    rp = kv.RopeParams.plain()
    ck1, cv1 = torch.zeros_like(d.cache_k), torch.zeros_like(d.cache_v)
    out1 = kv.prefill(d.q, d.k, d.v, d.positions, ck1, cv1, rp)
    ck2, cv2 = torch.zeros_like(d.cache_k), torch.zeros_like(d.cache_v)
    outs = []
    for i in range(t):
        lens = torch.full((n,), i, dtype=torch.int32, device="cuda")
        outs.append(kv.decode(d.q[:, i:i + 1].contiguous(), d.k[:, i:i + 1].contiguous(),
                              d.v[:, i:i + 1].contiguous(), d.positions[:, i].contiguous(),
                              ck2, cv2, lens, i, rp))
    torch.cuda.synchronize()
    out2 = torch.cat(outs, dim=1)
    assert torch.equal(ck1, ck2) and torch.equal(cv1, cv2)
    diff = (out1.double() - out2.double()).abs().max().item()
    assert diff <= 2e-3, diff


def test_deterministic(kv):
    cfg = custom(2, 70, 12, 2, 90, seed=800)
    inp = W.make_inputs(cfg, lens=np.array([3, 10], np.int32))
    rp = kv.RopeParams.plain()
    res = []
    for _ in range(2):
        d = to_dev(inp)
        o1 = kv.prefill_kv(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, 10, rp)
        o2 = kv.decode(d.q[:, :1].contiguous(), d.k[:, :1].contiguous(), d.v[:, :1].contiguous(),
                       (d.lens + 70).contiguous(), d.cache_k, d.cache_v, (d.lens + 70).contiguous(),
                       80, rp)
        torch.cuda.synchronize()
        res.append((o1.clone(), o2.clone(), d.cache_k.clone()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


def test_out_of_range_length_yields_nan_and_no_write(kv):
    """A device length above the host bound: the kernels skip that unit (no cache write,
    NaN output) and leave the other units correct."""
    lens = [5, 9]
    cfg = W.Config("custom", "decode", 2, 1, 1, 12, 2, 128, W.PLAIN_128, 0, 0, 20, 900, "")
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    d = to_dev(inp)
    bad = torch.tensor([5, 15], dtype=torch.int32, device="cuda")   # 15 > max_len = 9
    ck0 = d.cache_k.clone()
    out = kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, bad, 9, kv.RopeParams.plain())
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all() and torch.isfinite(out[0]).all()
    assert torch.equal(d.cache_k[1], ck0[1])
    # prefill_kv
    cfgp = custom(2, 8, 12, 2, 30, seed=901)
    inp = W.make_inputs(cfgp, lens=np.array([4, 6], np.int32))
    d = to_dev(inp)
    ck0 = d.cache_k.clone()
    badh = torch.tensor([4, 25], dtype=torch.int32, device="cuda")
    out = kv.prefill_kv(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, badh, 6,
                        kv.RopeParams.plain())
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all() and torch.isfinite(out[0]).all()
    assert torch.equal(d.cache_k[1], ck0[1])


def test_measurement_probes_run(kv):
    """The ceiling probes bench.py reports: the stream and plain-read probes read without
    error, and the MFMA probe records a shader clock between 0.5 and 3 GHz."""
    from kv_cache_causal_rope_amd import probes
    cfg = custom(3, 1, 12, 2, 300, seed=900)
    inp = W.make_inputs(cfg, lens=np.array([0, 150, 299], np.int32))
    d = to_dev(inp)
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    probes.stream_rows(d.cache_k, d.cache_v, d.lens, 299, 128, sink)
    probes.read(d.cache_k, 64, sink)
    blocks = 8
    clk = torch.zeros(4 + 4 * blocks, dtype=torch.int64, device="cuda")
    probes.mfma(blocks, 256, clk)
    torch.cuda.synchronize()
    c = clk[4:].view(blocks, 4).cpu().double()
    assert bool((c[:, 1] > c[:, 0]).all()) and bool((c[:, 3] > c[:, 2]).all())
    mhz = float(((c[:, 3] - c[:, 2]) / (c[:, 1] - c[:, 0])).mean()) * 100.0
    assert 500.0 < mhz < 3000.0, mhz


# ------------------------------------------------------------------ streams and threads
def test_decode_on_a_side_stream(kv):
    """Decode launched on a stream other than torch's current one, with the output and
    workspace allocated by the binding: the result matches the oracle even when the
    current stream is kept busy with fresh allocations meanwhile."""
    lens = [3000, 1200, 4000]
    cfg = W.Config("custom", "decode", 3, 1, 1, 12, 2, 128, W.PLAIN_128, 0, 0, 4100, 950, "")
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    _, ref64, _ = oracle.decode(bits(inp.q)[:, 0], bits(inp.k)[:, 0], bits(inp.v)[:, 0],
                                inp.positions.numpy()[:, 0], rk, rv, inp.lens.numpy(), cfg.scale,
                                ora_rope(cfg.rope))
    d = to_dev(inp)
    caches = [(d.cache_k.clone(), d.cache_v.clone()) for _ in range(4)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())      # the copies above are on the current stream
    outs = []
    for ck, cv in caches:
        outs.append(kv.decode(d.q, d.k, d.v, d.positions, ck, cv, d.lens, max(lens), kv.RopeParams.plain(),
                              stream=side))
        junk = torch.full((1 << 22,), 3.0, device="cuda")      # reuses freed blocks at once
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for o in outs:
        P.check_attention(bits(o)[:, 0], ref64, "decode on a side stream")


def test_profile_hook_is_per_thread(kv):
    """A hook set on one thread is recorded by that thread's next call only: a call on
    another thread neither records nor clears it, and that thread's own hook is its own.
    The events are first recorded around a GPU sleep of ~50 ms; a re-record around a
    decode kernel brings their interval down to well under a millisecond."""
    import threading
    cfg = W.Config("custom", "decode", 2, 1, 1, 12, 2, 128, W.PLAIN_128, 0, 0, 600, 960, "")
    d = to_dev(W.make_inputs(cfg, lens=np.array([500, 300], np.int32)))
    rp = kv.RopeParams.plain()

    def events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        evs[0].record()
        torch.cuda._sleep(100_000_000)
        evs[1].record()
        return evs

    mine, theirs = events(), events()
    torch.cuda.synchronize()
    assert mine[0].elapsed_time(mine[1]) > 10.0 and theirs[0].elapsed_time(theirs[1]) > 10.0
    kv.set_profile_events(mine[0], mine[1])
    errors = []

    def other():
        try:
            torch.cuda.set_device(0)
            kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, 500, rp)   # no hook here
            kv.set_profile_events(theirs[0], theirs[1])
            kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, 500, rp)
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    assert mine[0].elapsed_time(mine[1]) > 10.0          # untouched by the other thread
    assert theirs[0].elapsed_time(theirs[1]) < 1.0       # recorded by its own call there
    kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, 500, rp)
    torch.cuda.synchronize()
    assert mine[0].elapsed_time(mine[1]) < 1.0           # recorded by this thread's call


# ------------------------------------------------------------------ per-unit parameter sets
def _set_batch():
    """Layers of two kinds in one batch (ds4.c study notes, Part 4 sec. 1, Trace 2): plain
    RoPE with base 1e4, and "compressed" layers with their own base and scale and the YaRN
    ramp on (the rotated width is shared by all sets: the whole head here)."""
    plain = W.PLAIN_128
    compressed = W.Rope(base=160000.0, n_rot=128, yarn=True, freq_scale=1.0 / 16, ext_factor=1.0,
                        n_ctx_orig=65536, beta_fast=32.0, beta_slow=1.0, mscale=1.0 + 0.1 * np.log(16.0))
    return [plain, compressed]


def _kv_sets(kv, sets, unit_set):
    rp = kv.RopeParams.from_fields(sets[0])
    return rp.with_sets([kv.RopeParams.from_fields(s) for s in sets],
                        torch.tensor(unit_set, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("lens", [[0, 0, 0, 0, 0], [37, 0, 300, 64, 5]])
def test_parameter_sets_prefill_kv(kv, lens):
    sets, unit_set = _set_batch(), [1, 0, 1, 1, 0]
    n, t, hq, hkv = 5, 70, 12, 2
    cfg = custom(n, t, hq, hkv, max(lens) + t + 3, seed=970)
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    ref = oracle.prefill_kv(bits(inp.q), bits(inp.k), bits(inp.v), inp.positions.numpy(), rk, rv,
                            inp.lens.numpy(), cfg.scale, [ora_rope(s) for s in sets], np.array(unit_set))
    d = to_dev(inp)
    rp = _kv_sets(kv, sets, unit_set)
    if max(lens) == 0:
        out = kv.prefill(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, rp, scale=cfg.scale)
    else:
        out = kv.prefill_kv(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, max(lens), rp,
                            scale=cfg.scale)
    torch.cuda.synchronize()
    check_prefill(d, out, (ref[0], ref[1], ref[2], rk, rv), lens, t, f"parameter sets {lens}")


def test_parameter_sets_decode_and_rope_apply(kv):
    sets, unit_set = _set_batch(), [0, 1, 1, 0]
    lens = [900, 20000, 4097, 3]
    d, out, ref = None, None, None
    cfg = W.Config("custom", "decode", 4, 1, 1, 32, 8, 128, W.PLAIN_128, 0, 0, 20005, 980, "")
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    ora_sets = [ora_rope(s) for s in sets]
    ref = oracle.decode(bits(inp.q)[:, 0], bits(inp.k)[:, 0], bits(inp.v)[:, 0], inp.positions.numpy()[:, 0],
                        rk, rv, inp.lens.numpy(), cfg.scale, ora_sets, np.array(unit_set))
    d = to_dev(inp)
    rp = _kv_sets(kv, sets, unit_set)
    out = kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, max(lens), rp, scale=cfg.scale)
    torch.cuda.synchronize()
    check_decode(d, out, (ref[0], ref[1], ref[2], rk, rv), lens, "decode with parameter sets")
    # rope_apply: unit u of x [n, t, h, 128] rotates with its set
    g = torch.Generator().manual_seed(981)
    x = torch.randn((4, 9, 3, 128), generator=g).half()
    pos = torch.randint(0, 30000, (4, 9), generator=g, dtype=torch.int32)
    ref_bits = np.empty(bits(x).shape, np.uint16)
    ref64 = np.empty(ref_bits.shape)
    for u in range(4):
        ref_bits[u], ref64[u] = oracle.rope(bits(x)[u], pos.numpy()[u], ora_sets[unit_set[u]])
    xd = x.cuda()
    kv.rope_apply(xd, pos.cuda(), rp)
    torch.cuda.synchronize()
    P.check_k_rows(bits(xd), ref_bits, ref64, "rope_apply with parameter sets")


def test_invalid_parameter_set_index_gives_nan_rotation(kv):
    sets = _set_batch()
    cfg = custom(2, 8, 12, 2, 8, seed=985)
    d = to_dev(W.make_inputs(cfg, lens=np.zeros(2, np.int32)))
    rp = _kv_sets(kv, sets, [1, 7])
    out = kv.prefill(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, rp, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0]).all() and torch.isnan(out[1]).all()
    assert torch.isnan(d.cache_k[1]).all() and torch.isfinite(d.cache_v[1]).all()


# ------------------------------------------------------------------ phase consistency, long positions
def test_gpu_prefill_kv_equals_successive_gpu_decodes_near_32k(kv):
    """The K rows the prefill side writes (rope_append) and those the decode prologue
    writes agree bit for bit at positions just below 32k, where the angle reduction is
    hardest (plain and YaRN tail rotation)."""
    for rope in (W.PLAIN_128, W.YARN_TAIL_64):
        n, t, hq, hkv, hist = 2, 24, 32, 8, 32700
        cfg = custom(n, t, hq, hkv, hist + t, rope=rope, seed=990)
        inp = W.make_inputs(cfg, lens=np.full(n, hist, np.int32))
        d = to_dev(inp)
        rp = kv.RopeParams.from_fields(rope)
        ck1, cv1 = d.cache_k.clone(), d.cache_v.clone()
        out1 = kv.prefill_kv(d.q, d.k, d.v, d.positions, ck1, cv1, d.lens, hist, rp)
        ck2, cv2 = d.cache_k.clone(), d.cache_v.clone()
        outs = []
        for i in range(t):
            lens = torch.full((n,), hist + i, dtype=torch.int32, device="cuda")
            outs.append(kv.decode(d.q[:, i:i + 1].contiguous(), d.k[:, i:i + 1].contiguous(),
                                  d.v[:, i:i + 1].contiguous(), d.positions[:, i].contiguous(),
                                  ck2, cv2, lens, hist + i, rp))
        torch.cuda.synchronize()
        assert torch.equal(ck1.view(torch.int16), ck2.view(torch.int16)), rope
        assert torch.equal(cv1.view(torch.int16), cv2.view(torch.int16))
        diff = (out1.double() - torch.cat(outs, dim=1).double()).abs().max().item()
        assert diff <= 2e-3, diff
