"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Every output row of every workload is compared with the oracle, computed on host copies
of the inputs taken before the GPU call (no oracle input comes from the GPU path):
  * the T = 1024 28-layer prefill and the 3840 + 256 32-layer prefill_kv: the oracle's
    prefill_kv over all units;
  * the three 28-layer decode workloads: the oracle's decode over all units;
  * the YaRN 32k batch-64 decode: the GPU runs all 4 layers in one call; the oracle runs
    one layer (64 units) at a time, to bound host memory.
Checked: every output row within 2e-3 absolute / 1e-2 row-relative; every appended K row
equal to the oracle's f16 rounding of its fp64 rotation (boundary rule in
tests/parity.py) and every appended V row bit-identical; every other cache row unchanged
(compared on the GPU against a copy taken before the call).
"""
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


def ora_rope(r):
    return oracle.RopeParams(base=r.base, n_rot=r.n_rot, yarn=r.yarn, freq_scale=r.freq_scale,
                             ext_factor=r.ext_factor, n_ctx_orig=r.n_ctx_orig,
                             beta_fast=r.beta_fast, beta_slow=r.beta_slow, mscale=r.mscale)


bits = P.to_np_bits


def appended_rows(cache, lens_dev, t):
    """Rows lens[u] .. lens[u] + t - 1 of every (unit, KV head): [n, t, hkv, d]."""
    n, hkv, _, d = cache.shape
    idx = lens_dev.long().view(n, 1) + torch.arange(t, device=cache.device).view(1, t)
    gather = idx.view(n, 1, t, 1).expand(n, hkv, t, d)
    return torch.gather(cache, 2, gather).permute(0, 2, 1, 3).contiguous()


def check_untouched(cache, cache0, lens_dev, t, what, chunk=16):
    """Every row outside [lens[u], lens[u] + t) equal, bit for bit, to the copy taken
    before the call (on the GPU, a few units at a time)."""
    n, hkv, s_cap, _ = cache.shape
    rows = torch.arange(s_cap, device=cache.device).view(1, 1, s_cap)
    for u0 in range(0, n, chunk):
        u1 = min(n, u0 + chunk)
        lo = lens_dev[u0:u1].long().view(-1, 1, 1)
        new = (rows >= lo) & (rows < lo + t)
        diff = (cache[u0:u1].view(torch.int16) != cache0[u0:u1].view(torch.int16)).any(-1)
        bad = diff & ~new
        assert not bool(bad.any()), f"{what}: cache rows outside the appended ones changed"


def report(cfg, max_abs, row_rel, kb, rows, prof):
    print(f"{cfg.name}: {rows} output rows (all), max abs {max_abs:.2e} (at |ref| "
          f"{prof['ref_at_max_abs']:.3f}, index {prof['where']}), "
          f"row-rel {row_rel:.2e}, K boundary cases {kb}", flush=True)


def run_prefill(kv, cfg):
    inp = W.make_inputs(cfg, device="cuda")
    lens = inp.lens.cpu().numpy()
    host = {x: bits(getattr(inp, x)) for x in ("q", "k", "v", "cache_k", "cache_v")}
    pos = inp.positions.cpu().numpy()
    ck0, cv0 = inp.cache_k.clone(), inp.cache_v.clone()
    rp = kv.RopeParams.from_fields(cfg.rope)
    if cfg.phase == "prefill":
        out = kv.prefill(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, rp,
                         scale=cfg.scale)
    else:
        out = kv.prefill_kv(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, inp.lens,
                            int(lens.max()), rp, scale=cfg.scale)
    torch.cuda.synchronize()
    rk, rv = host["cache_k"].copy(), host["cache_v"].copy()
    _, ref64, k64 = oracle.prefill_kv(host["q"], host["k"], host["v"], pos, rk, rv, lens, cfg.scale,
                                      ora_rope(cfg.rope))
    max_abs, row_rel = P.check_attention(bits(out), ref64, cfg.name)
    prof = P.error_profile(bits(out), ref64)
    t = cfg.t
    gk = bits(appended_rows(inp.cache_k, inp.lens, t))
    gv = bits(appended_rows(inp.cache_v, inp.lens, t))
    n = cfg.n
    ok_rows = np.stack([rk[u][:, lens[u]:lens[u] + t].transpose(1, 0, 2) for u in range(n)])
    ov_rows = np.stack([rv[u][:, lens[u]:lens[u] + t].transpose(1, 0, 2) for u in range(n)])
    assert np.array_equal(gv, ov_rows), f"{cfg.name}: appended V rows differ"
    kb = P.check_k_rows(gk, ok_rows, k64, cfg.name + " appended K")
    check_untouched(inp.cache_k, ck0, inp.lens, t, cfg.name + " K")
    check_untouched(inp.cache_v, cv0, inp.lens, t, cfg.name + " V")
    report(cfg, max_abs, row_rel, kb, n * t * cfg.hq, prof)


def run_decode(kv, cfg, units_per_oracle_call=None):
    inp = W.make_inputs(cfg, device="cuda")
    lens = inp.lens.cpu().numpy()
    n = cfg.n
    step = units_per_oracle_call or n
    host_q, host_k, host_v = bits(inp.q)[:, 0], bits(inp.k)[:, 0], bits(inp.v)[:, 0]
    pos = inp.positions.cpu().numpy()[:, 0]
    # host copies of the caches, one slice of units at a time
    host_ck = [bits(inp.cache_k[u0:u0 + step]) for u0 in range(0, n, step)]
    host_cv = [bits(inp.cache_v[u0:u0 + step]) for u0 in range(0, n, step)]
    ck0, cv0 = inp.cache_k.clone(), inp.cache_v.clone()
    rp = kv.RopeParams.from_fields(cfg.rope)
    out = kv.decode(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, inp.lens,
                    int(lens.max()), rp, scale=cfg.scale)
    torch.cuda.synchronize()
    got = bits(out)[:, 0]
    gk = bits(appended_rows(inp.cache_k, inp.lens, 1))[:, 0]
    gv = bits(appended_rows(inp.cache_v, inp.lens, 1))[:, 0]
    check_untouched(inp.cache_k, ck0, inp.lens, 1, cfg.name + " K")
    check_untouched(inp.cache_v, cv0, inp.lens, 1, cfg.name + " V")
    del ck0, cv0
    max_abs = row_rel = 0.0
    prof = {"ref_at_max_abs": 0.0, "where": None}
    kb = 0
    for i, u0 in enumerate(range(0, n, step)):
        u1 = min(n, u0 + step)
        rk, rv = host_ck[i], host_cv[i]
        _, ref64, k64 = oracle.decode(host_q[u0:u1], host_k[u0:u1], host_v[u0:u1], pos[u0:u1], rk, rv,
                                      lens[u0:u1], cfg.scale, ora_rope(cfg.rope))
        what = f"{cfg.name} units {u0}..{u1 - 1}"
        a, r = P.check_attention(got[u0:u1], ref64, what)
        pr = P.error_profile(got[u0:u1], ref64)
        if a >= max_abs and pr["where"] is not None:
            prof = {"ref_at_max_abs": pr["ref_at_max_abs"],
                    "where": (pr["where"][0] + u0,) + pr["where"][1:]}
        max_abs, row_rel = max(max_abs, a), max(row_rel, r)
        ok_rows = np.stack([rk[u - u0][:, lens[u]] for u in range(u0, u1)])
        ov_rows = np.stack([rv[u - u0][:, lens[u]] for u in range(u0, u1)])
        assert np.array_equal(gv[u0:u1], ov_rows), f"{what}: appended V rows differ"
        kb += P.check_k_rows(gk[u0:u1], ok_rows, k64, what + " appended K")
        host_ck[i] = host_cv[i] = None
    report(cfg, max_abs, row_rel, kb, n * cfg.hq, prof)


@pytest.mark.timeout(300)
def test_full_qwen_prefill_1024(kv):
    run_prefill(kv, W.CONFIGS["qwen1p5b_prefill_t1024"])


@pytest.mark.timeout(300)
def test_full_prefill_kv_3840_plus_256(kv):
    run_prefill(kv, W.CONFIGS["h4096_prefill_kv_3840p256"])


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["qwen1p5b_decode_l1024_b1", "qwen1p5b_decode_l4096_b1",
                                  "qwen1p5b_decode_l4096_b32"])
def test_full_qwen_decode(kv, name):
    run_decode(kv, W.CONFIGS[name])


@pytest.mark.timeout(600)
def test_full_yarn_decode_32k(kv):
    run_decode(kv, W.CONFIGS["yarn_decode_l32k_b64"], units_per_oracle_call=64)
    torch.cuda.empty_cache()
