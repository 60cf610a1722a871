"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The GPU runs the whole workload; the oracle recomputes a sample of it one output row at
a time (it cannot afford every row of the large workloads).  Host copies of every input
the oracle reads are taken before the GPU call, so no oracle input comes from the GPU
path.  Checked at full size:
  * sampled output rows (unit, token, head) within 2e-3 absolute / 1e-2 row-relative;
  * every appended K row of every unit equal to the oracle's f16 rounding of its fp64
    rotation (boundary rule in tests/parity.py), every appended V row bit-identical;
  * all outputs finite.
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


def bits(x):
    return P.to_np_bits(x)


def check_appended_rows(cfg, inp_host_k, pos_host, lens_host, ck_dev, cv_dev, v_dev):
    """Every unit's appended rows: K by the rounding rule, V bit-identical."""
    n, t, hkv, d = inp_host_k.shape
    rk_bits, rk64 = oracle.rope(bits(inp_host_k).reshape(n * t, hkv, d),
                                pos_host.reshape(-1), ora_rope(cfg.rope))
    rk_bits = rk_bits.reshape(n, t, hkv, d)
    rk64 = rk64.reshape(n, t, hkv, d)
    idx = torch.from_numpy(lens_host.astype(np.int64)).cuda().view(n, 1) + \
        torch.arange(t, device="cuda").view(1, t)                       # [n, t] rows
    gather = idx.view(n, 1, t, 1).expand(n, hkv, t, d)
    gk = torch.gather(ck_dev, 2, gather).permute(0, 2, 1, 3).contiguous()  # [n, t, hkv, d]
    gv = torch.gather(cv_dev, 2, gather).permute(0, 2, 1, 3).contiguous()
    assert torch.equal(gv.view(torch.int16), v_dev.view(torch.int16)), "appended V rows differ"
    return P.check_k_rows(bits(gk), rk_bits, rk64, cfg.name + " appended K")


def sample_rows(rng, n, t, hq, count, must=()):
    rows = {tuple(m) for m in must}
    while len(rows) < count:
        rows.add((int(rng.integers(n)), int(rng.integers(t)), int(rng.integers(hq))))
    return sorted(rows)


def oracle_rows(cfg, rows, host, caches_after):
    """Recompute output rows one by one: rotated q (oracle), attention over rows
    0 .. len + token of the oracle-appended caches."""
    units = np.array([r[0] for r in rows], np.int32)
    toks = np.array([r[1] for r in rows], np.int32)
    heads = np.array([r[2] for r in rows], np.int32)
    ck, cv, unit_index = caches_after
    qsel = bits(host["q"])[units, toks, heads][:, None, :]              # [ns, 1, d]
    psel = host["pos"][units, toks]
    qrot, _ = oracle.rope(qsel, psel, ora_rope(cfg.rope))
    lens = host["lens"][units] + toks
    return oracle.decode_rows(qrot[:, 0, :].copy(), ck, cv, unit_index[units], heads, lens,
                              cfg.hq, cfg.scale)


def host_caches_after_append(cfg, host, units):
    """Host copies of the sampled units' caches with the oracle's own append."""
    sel = np.array(sorted(set(units)), np.int32)
    ck = bits(host["cache_k"][sel]).copy()
    cv = bits(host["cache_v"][sel]).copy()
    n_t = host["k"].shape[1]
    krot, _ = oracle.rope(bits(host["k"][sel]).reshape(len(sel) * n_t, cfg.hkv, cfg.d),
                          host["pos"][sel].reshape(-1), ora_rope(cfg.rope))
    oracle.append(ck, cv, krot.reshape(len(sel), n_t, cfg.hkv, cfg.d), bits(host["v"][sel]),
                  host["lens"][sel])
    unit_index = np.full(cfg.n, -1, np.int32)
    unit_index[sel] = np.arange(len(sel), dtype=np.int32)
    return ck, cv, unit_index


def run_full(kv, cfg, nsample, seed=1234):
    inp = W.make_inputs(cfg, device="cuda")
    rng = np.random.default_rng(seed)
    n, t = cfg.n, cfg.t
    lens = inp.lens.cpu().numpy()
    must = [(0, 0, 0), (n - 1, t - 1, cfg.hq - 1), (int(np.argmax(lens)), t - 1, 0),
            (int(np.argmin(lens)), 0, cfg.hq // 2)]
    rows = sample_rows(rng, n, t, cfg.hq, nsample, must)
    units = sorted({r[0] for r in rows})
    ut = torch.tensor(units, device="cuda")
    host = {"q": inp.q.cpu(), "k": inp.k.cpu(), "v": inp.v.cpu(),
            "pos": inp.positions.cpu().numpy(), "lens": lens,
            "cache_k": inp.cache_k.index_select(0, ut).cpu(),
            "cache_v": inp.cache_v.index_select(0, ut).cpu()}
    # the sampled units' caches are indexed by position in `units`
    remap = {u: i for i, u in enumerate(units)}
    host_local = dict(host)
    host_local["q"] = host["q"][units]
    host_local["k"] = host["k"][units]
    host_local["v"] = host["v"][units]
    host_local["pos"] = host["pos"][units]
    host_local["lens"] = lens[units]
    cfg_local = W.Config(cfg.name, cfg.phase, len(units), 1, t, cfg.hq, cfg.hkv, cfg.d, cfg.rope,
                         cfg.len_lo, cfg.len_hi, cfg.s_cap, cfg.seed, "")
    ck, cv, uidx = host_caches_after_append(cfg_local, host_local, list(range(len(units))))
    rows_local = [(remap[u], tt, h) for (u, tt, h) in rows]

    rp = kv.RopeParams.from_fields(cfg.rope)
    if cfg.phase == "decode":
        out = kv.decode(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, inp.lens,
                        int(lens.max()), rp, scale=cfg.scale)
    elif cfg.phase == "prefill":
        out = kv.prefill(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, rp,
                         scale=cfg.scale)
    else:
        out = kv.prefill_kv(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, inp.lens,
                            int(lens.max()), rp, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), f"{cfg.name}: non-finite outputs"

    ref = oracle_rows(cfg_local, rows_local, host_local, (ck, cv, uidx))
    got = np.stack([bits(out[u, tt, h]) for (u, tt, h) in rows])
    max_abs, row_rel = P.check_attention(got, ref, cfg.name)
    nb = check_appended_rows(cfg, host["k"], host["pos"], lens, inp.cache_k, inp.cache_v, inp.v)
    print(f"{cfg.name}: {len(rows)} sampled rows, max abs {max_abs:.2e}, row-rel {row_rel:.2e}, "
          f"K boundary cases {nb}")
    return out


@pytest.mark.timeout(300)
def test_full_qwen_prefill_1024(kv):
    run_full(kv, W.CONFIGS["qwen1p5b_prefill_t1024"], 96)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["qwen1p5b_decode_l1024_b1", "qwen1p5b_decode_l4096_b1",
                                  "qwen1p5b_decode_l4096_b32"])
def test_full_qwen_decode(kv, name):
    run_full(kv, W.CONFIGS[name], 64)


@pytest.mark.timeout(300)
def test_full_prefill_kv_3840_plus_256(kv):
    run_full(kv, W.CONFIGS["h4096_prefill_kv_3840p256"], 96)


@pytest.mark.timeout(600)
def test_full_yarn_decode_32k(kv):
    run_full(kv, W.CONFIGS["yarn_decode_l32k_b64"], 24)
    torch.cuda.empty_cache()
