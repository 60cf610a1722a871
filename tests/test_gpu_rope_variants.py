"""GPU parity of the rotation variants against the CPU oracle: half-split pairing (pair j
= dims (o + j, o + j + n_rot/2)), the inverse rotation (sine's sign flipped) and caller
tables of cos / sin gathered by position, through every entry point that rotates
(rope_apply, prefill, prefill_kv, decode).  Same bars as the plain-rotation parity tests
(tests/parity.py): attention within 2e-3 absolute and 1e-2 row-relative of the oracle's
fp64 output, V and untouched cache rows bit-identical, rotated K rows equal to the
oracle's f16 rounding.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from kv_cache_causal_rope_amd import workloads as W
from tests import parity as P
from tests.test_gpu_parity import (bits, check_decode, check_prefill, custom, kv, ora_rope,  # noqa: F401
                                   to_dev)

pytestmark = pytest.mark.gpu

HALF_32 = W.Rope(n_rot=32)
HALF_96 = W.Rope(n_rot=96, base=500000.0)


def make_tables(rope: W.Rope, rows: int, stretch: float = 1.37):
    """cos / sin of a schedule other than the computed one (angles stretched), so a kernel
    that ignored the tables would fail; float32 [rows, n_rot / 2]."""
    half = rope.n_rot // 2
    j = np.arange(half)
    ang = np.arange(rows)[:, None] * np.power(rope.base, -2.0 * j / rope.n_rot)[None, :] * stretch
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Variant:
    half_split: bool = False
    inverse: bool = False
    table_rows: int = 0  # 0: computed angles

    def name(self):
        return "".join([("half" if self.half_split else "adj"), ("-inv" if self.inverse else ""),
                        (f"-tab{self.table_rows}" if self.table_rows else "")])


def params(kv, rope: W.Rope, var: Variant):
    """(oracle params, library params) of one variant; tables built once for both."""
    ora = ora_rope(rope).replace(half_split=var.half_split, inverse=var.inverse)
    lib = kv.RopeParams.from_fields(rope)
    if var.table_rows:
        ct, st = make_tables(rope, var.table_rows)
        ora = ora.replace(cos_table=ct, sin_table=st)
        lib = lib.with_variant(var.half_split, var.inverse, torch.from_numpy(ct).cuda(),
                               torch.from_numpy(st).cuda())
    else:
        lib = lib.with_variant(var.half_split, var.inverse)
    return ora, lib


VARIANTS = [Variant(True), Variant(False, True), Variant(True, True), Variant(False, False, 6000),
            Variant(True, True, 6000)]


@pytest.mark.parametrize("rope", [W.PLAIN_128, W.YARN_TAIL_64, HALF_32, HALF_96],
                         ids=["plain128", "yarn64", "n32", "n96"])
@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: v.name())
def test_rope_apply_variants(kv, rope, var):
    g = torch.Generator().manual_seed(31)
    n, t, h = 2, 41, 5
    x = torch.randn((n, t, h, 128), generator=g).half()
    pos = torch.randint(0, 6000, (n, t), generator=g, dtype=torch.int32)
    ora, lib = params(kv, rope, var)
    ref_bits, ref64 = oracle.rope(bits(x).reshape(n * t, h, 128), pos.numpy().reshape(-1), ora)
    xd = x.cuda()
    kv.rope_apply(xd, pos.cuda(), lib)
    torch.cuda.synchronize()
    P.check_k_rows(bits(xd).reshape(n * t, h, 128), ref_bits, ref64, f"rope_apply {var.name()}")


def test_rope_apply_table_out_of_range_is_nan(kv):
    rope = W.YARN_TAIL_64
    var = Variant(True, False, 100)
    g = torch.Generator().manual_seed(32)
    x = torch.randn((1, 6, 3, 128), generator=g).half()
    pos = torch.tensor([[0, 99, 100, -1, 5000, 7]], dtype=torch.int32)
    ora, lib = params(kv, rope, var)
    ref_bits, ref64 = oracle.rope(bits(x).reshape(6, 3, 128), pos.numpy().reshape(-1), ora)
    xd = x.cuda()
    kv.rope_apply(xd, pos.cuda(), lib)
    torch.cuda.synchronize()
    got = bits(xd).reshape(6, 3, 128)
    bad = np.array([False, False, True, True, True, False])
    gf = got.view(np.float16)
    assert np.isnan(gf[bad][..., 64:]).all() and np.isnan(ref64[bad][..., 64:]).all()
    assert np.array_equal(got[..., :64], ref_bits[..., :64])
    P.check_k_rows(got[~bad], ref_bits[~bad], ref64[~bad], "rope_apply table in range")


def run_prefill_variant(kv, cfg, lens, rope, var):
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    ora, lib = params(kv, rope, var)
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    ref = oracle.prefill_kv(bits(inp.q), bits(inp.k), bits(inp.v), inp.positions.numpy(), rk, rv,
                            inp.lens.numpy(), cfg.scale, ora)
    d = to_dev(inp)
    out = kv.prefill_kv(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, int(max(lens)), lib,
                        scale=cfg.scale)
    torch.cuda.synchronize()
    return d, out, (*ref, rk, rv)


@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: v.name())
@pytest.mark.parametrize("n,t,hq,hkv,lens,rope", [
    (2, 77, 12, 2, [0, 0], W.PLAIN_128),        # G = 6: rotation factors shared in LDS
    (1, 130, 8, 4, [0], W.PLAIN_128),           # G = 2: per-lane rotation
    (2, 45, 32, 8, [37, 300], W.YARN_TAIL_64),  # G = 4 with history, tail rotation
    (1, 64, 12, 2, [20], HALF_96),              # n_rot 96
    (2, 50, 6, 2, [0, 9], HALF_32),             # n_rot 32, G = 3
], ids=["g6", "g2", "yarn-hist", "n96", "n32"])
def test_prefill_variants(kv, var, n, t, hq, hkv, lens, rope):
    cfg = custom(n, t, hq, hkv, max(lens) + t + 5, rope=rope, seed=800 + t)
    d, out, ref = run_prefill_variant(kv, cfg, lens, rope, var)
    check_prefill(d, out, ref, lens, t, f"prefill {var.name()} n{n} t{t} {hq}/{hkv} {lens}")


@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: v.name())
@pytest.mark.parametrize("n,hq,hkv,lens,rope", [
    (4, 12, 2, [0, 63, 300, 1700], W.PLAIN_128),
    (3, 32, 8, [700, 31, 5000], W.YARN_TAIL_64),
    (2, 4, 4, [90, 2], HALF_96),
], ids=["g6", "yarn", "n96"])
def test_decode_variants(kv, var, n, hq, hkv, lens, rope):
    cfg = W.Config("custom", "decode", n, 1, 1, hq, hkv, 128, rope, 0, 0, max(lens) + 3, 900 + n, "")
    inp = W.make_inputs(cfg, lens=np.asarray(lens, np.int32))
    ora, lib = params(kv, rope, var)
    rk, rv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    ref = oracle.decode(bits(inp.q)[:, 0], bits(inp.k)[:, 0], bits(inp.v)[:, 0], inp.positions.numpy()[:, 0],
                        rk, rv, inp.lens.numpy(), cfg.scale, ora)
    d = to_dev(inp)
    out = kv.decode(d.q, d.k, d.v, d.positions, d.cache_k, d.cache_v, d.lens, int(max(lens)), lib,
                    scale=cfg.scale)
    torch.cuda.synchronize()
    check_decode(d, out, (*ref, rk, rv), lens, f"decode {var.name()} {hq}/{hkv} {lens}")


def test_half_split_rejects_unsupported_width(kv):
    x = torch.zeros((1, 1, 1, 128), dtype=torch.float16, device="cuda")
    pos = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(kv.KVRopeError):
        kv.rope_apply(x, pos, kv.RopeParams.plain(n_rot=48).with_variant(half_split=True))
