"""attn_decode_noalloc, called through the C ABI: the allocation-free decode gives the
same outputs and cache rows as attn_decode with a caller workspace, bit for bit, on two
calls in a row, the second with a smaller input (its scratch then holds the first call's
partials), and rejects shapes whose workspace exceeds its scratch."""
import ctypes

import numpy as np
import pytest
import torch

from kv_cache_causal_rope_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    import kv_cache_causal_rope_amd as kv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kv.lib()
    return kv


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _inputs(n, hq, hkv, lens, s_cap, rope, seed):
    cfg = W.Config("noalloc", "decode", n, 1, 1, hq, hkv, 128, rope, 0, 0, s_cap, seed, "")
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32), device="cuda")
    return cfg, inp


def _decode_with_workspace(kv, cfg, inp, ck, cv, rp, max_len):
    n = cfg.n
    out = torch.empty_like(inp.q)
    need = kv.workspace_size(n, cfg.hq, cfg.hkv, max_len)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    st = kv.lib().attn_decode(_ptr(inp.q), _ptr(inp.k), _ptr(inp.v), _ptr(inp.positions), _ptr(ck), _ptr(cv),
                              _ptr(inp.lens), max_len, _ptr(out), n, cfg.hq, cfg.hkv, 128, cfg.s_cap,
                              cfg.scale, ctypes.byref(rp), _ptr(ws), ws.numel(), None)
    assert st == 0, kv.status_string(st)
    return out, need


def _decode_noalloc(kv, cfg, inp, ck, cv, rp, max_len):
    out = torch.empty_like(inp.q)
    st = kv.lib().attn_decode_noalloc(_ptr(inp.q), _ptr(inp.k), _ptr(inp.v), _ptr(inp.positions), _ptr(ck),
                                      _ptr(cv), _ptr(inp.lens), max_len, _ptr(out), cfg.n, cfg.hq, cfg.hkv,
                                      128, cfg.s_cap, cfg.scale, ctypes.byref(rp), None)
    assert st == 0, kv.status_string(st)
    return out


def test_noalloc_decode_matches_workspace_decode_twice(kv):
    cases = [  # the 28-layer batch-32 4k-row shape, then a smaller YaRN batch
        (896, 12, 2, W.PLAIN_128, 4097, 2048, 4096, 31),
        (12, 32, 8, W.YARN_TAIL_64, 9000, 100, 8999, 32),
    ]
    limit = kv.lib().attn_decode_noalloc_max_workspace()
    assert limit == 64 << 20
    for n, hq, hkv, rope, s_cap, lo, hi, seed in cases:
        lens = np.random.default_rng(seed).integers(lo, hi + 1, n)
        cfg, inp = _inputs(n, hq, hkv, lens, s_cap, rope, seed)
        rp = kv.RopeParams.from_fields(rope)
        max_len = int(lens.max())
        ck1, cv1 = inp.cache_k.clone(), inp.cache_v.clone()
        ref, need = _decode_with_workspace(kv, cfg, inp, ck1, cv1, rp, max_len)
        assert 0 < need <= limit
        ck2, cv2 = inp.cache_k.clone(), inp.cache_v.clone()
        got = _decode_noalloc(kv, cfg, inp, ck2, cv2, rp, max_len)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"outputs differ (n={n})"
        assert torch.equal(ck1.view(torch.int16), ck2.view(torch.int16))
        assert torch.equal(cv1.view(torch.int16), cv2.view(torch.int16))
        del inp, ck1, cv1, ck2, cv2
        torch.cuda.empty_cache()


def test_noalloc_decode_rejects_a_workspace_beyond_its_scratch(kv):
    L = kv.lib()
    limit = L.attn_decode_noalloc_max_workspace()
    # 64 units x 32 heads x 32k-row caches need more partials than the scratch holds
    n, hq, hkv, max_len = 1024, 32, 8, 32768
    assert kv.workspace_size(n, hq, hkv, max_len) > limit
    a, b = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    st = L.attn_decode_noalloc(a, a, a, a, b, b, a, max_len, b, n, hq, hkv, 128, max_len + 1, 0.088,
                               ctypes.byref(kv.RopeParams.plain()), None)
    assert st == kv.ATTN_ERR_WORKSPACE
