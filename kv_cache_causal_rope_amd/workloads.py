"""Workload table and seeded synthetic input generators.

This module holds shapes and random draws only -- none of the attention or rotary
arithmetic.  The same generators feed the GPU library and the CPU oracle.

Shapes follow the pages' workloads:
  * the Qwen-1.5B-style block of the Buddy-MLIR DeepSeek-R1-Distill walkthrough
    (sec. 6.4.1 / 6.4.3: 2 KV heads x head_dim 128, a 1024-row f16 cache per layer,
    28 layers) with 12 query heads;
  * the example block of the Sophgo MLIR-based LLM compilation paper (sec. 2.3, Fig. 2:
    hidden 4096, kv_head 2, head_dim 128 -> 32 query heads, 32 layers);
  * a long-context YaRN tail-rotation decode (ds4.c study notes, Part 4 sec. 1).

Every tensor value is i.i.d. N(0, 1) drawn as float32 and rounded to f16; lengths are
uniform integers.  Draw order per config: lengths, q, k, v, cache_k, cache_v.  Units are
numbered u = layer * batch + b; a sequence keeps its length across its layers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Rope:
    """Rotary settings as plain data (each side builds its own parameter struct)."""
    base: float = 10000.0
    n_rot: int = 128
    yarn: bool = False
    freq_scale: float = 1.0
    ext_factor: float = 0.0
    n_ctx_orig: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0


PLAIN_128 = Rope()
# YaRN tail rotation: scale factor 4 -> freq_scale 1/4, magnitude 1 + 0.1 ln 4.
YARN_TAIL_64 = Rope(base=10000.0, n_rot=64, yarn=True, freq_scale=0.25, ext_factor=1.0,
                    n_ctx_orig=4096, beta_fast=32.0, beta_slow=1.0,
                    mscale=1.0 + 0.1 * math.log(4.0))


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    phase: str           # "prefill" | "prefill_kv" | "decode"
    layers: int
    batch: int
    t: int               # new tokens per unit
    hq: int
    hkv: int
    d: int
    rope: Rope
    len_lo: int          # history length range [len_lo, len_hi] (per sequence)
    len_hi: int
    s_cap: int           # cache rows per (unit, kv head)
    seed: int
    description: str

    @property
    def n(self) -> int:
        return self.layers * self.batch

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


CONFIGS = {c.name: c for c in [
    Config("tiny_prefill_t64", "prefill", 1, 1, 64, 12, 2, 128, PLAIN_128, 0, 0, 64, 0,
           "1 layer, batch 1, T=64, 12q/2kv x 128, plain RoPE base 1e4"),
    Config("qwen1p5b_prefill_t1024", "prefill", 28, 1, 1024, 12, 2, 128, PLAIN_128, 0, 0,
           1024, 1, "28 layers, batch 1, T=1024, 12q/2kv x 128, cache [28,2,1024,128]"),
    Config("qwen1p5b_decode_l1024_b1", "decode", 28, 1, 1, 12, 2, 128, PLAIN_128, 512, 1024,
           1025, 2, "28 layers, batch 1, cache length U[512,1024]"),
    Config("qwen1p5b_decode_l4096_b1", "decode", 28, 1, 1, 12, 2, 128, PLAIN_128, 2048, 4096,
           4097, 3, "28 layers, batch 1, cache length U[2048,4096]"),
    Config("qwen1p5b_decode_l4096_b32", "decode", 28, 32, 1, 12, 2, 128, PLAIN_128, 2048,
           4096, 4097, 4, "28 layers, batch 32, cache length U[2048,4096]"),
    Config("h4096_prefill_kv_3840p256", "prefill_kv", 32, 1, 256, 32, 2, 128, PLAIN_128, 3840,
           3840, 4096, 5, "32 layers, batch 1, 3840 history + 256 new, 32q/2kv x 128"),
    Config("yarn_decode_l32k_b64", "decode", 4, 64, 1, 32, 8, 128, YARN_TAIL_64, 8192, 32768,
           32769, 6, "4 layers, batch 64, 32q/8kv x 128, YaRN tail 64 dims, U[8192,32768]"),
]}


def draw_lengths(gen: torch.Generator, cfg: Config) -> np.ndarray:
    """Per-unit history lengths (one draw per sequence, repeated over layers)."""
    seq = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.batch,), generator=gen,
                        dtype=torch.int64)
    lens = seq.repeat(cfg.layers)  # u = layer * batch + b
    return lens.to(torch.int32).numpy()


def randn_f16(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).half()


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor          # [n, t, hq, d] f16
    k: torch.Tensor          # [n, t, hkv, d] f16
    v: torch.Tensor          # [n, t, hkv, d] f16
    positions: torch.Tensor  # [n, t] int32
    lens: torch.Tensor       # [n] int32
    cache_k: torch.Tensor    # [n, hkv, s_cap, d] f16
    cache_v: torch.Tensor


def make_inputs(cfg: Config, *, n: Optional[int] = None, t: Optional[int] = None,
                s_cap: Optional[int] = None, lens: Optional[np.ndarray] = None,
                seed: Optional[int] = None, device: str = "cpu",
                poison_tail: bool = False) -> Inputs:
    """Seeded inputs for `cfg` (optionally with a smaller unit count / token count).

    History rows [0, len) of the caches hold N(0,1) values (treated as already rotated);
    rows >= len are zero, or NaN when `poison_tail` (to prove nothing reads past len).
    Positions of the new tokens are len, len+1, ..., len+t-1.
    """
    seed = cfg.seed if seed is None else seed
    n = cfg.n if n is None else n
    t = cfg.t if t is None else t
    s_cap = cfg.s_cap if s_cap is None else s_cap
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(seed)
    if lens is None:
        full = draw_lengths(cpu_gen, cfg)
        lens = np.resize(full, n).astype(np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    assert lens.shape == (n,)
    if np.any(lens.astype(np.int64) + t > s_cap):
        raise ValueError("cache capacity too small for lengths + new tokens")
    q = randn_f16(gen, (n, t, cfg.hq, cfg.d), device)
    k = randn_f16(gen, (n, t, cfg.hkv, cfg.d), device)
    v = randn_f16(gen, (n, t, cfg.hkv, cfg.d), device)
    cache_k = randn_f16(gen, (n, cfg.hkv, s_cap, cfg.d), device)
    cache_v = randn_f16(gen, (n, cfg.hkv, s_cap, cfg.d), device)
    lens_t = torch.from_numpy(lens).to(device)
    rows = torch.arange(s_cap, device=device).view(1, 1, s_cap, 1)
    tail = rows >= lens_t.view(n, 1, 1, 1).long()
    fill = float("nan") if poison_tail else 0.0
    cache_k.masked_fill_(tail, fill)
    cache_v.masked_fill_(tail, fill)
    positions = (lens_t.view(n, 1).long() + torch.arange(t, device=device).view(1, t))
    return Inputs(q, k, v, positions.to(torch.int32).contiguous(), lens_t.contiguous(),
                  cache_k, cache_v)


def bits(x: torch.Tensor) -> np.ndarray:
    """f16 tensor (any device) -> host numpy uint16 bit patterns."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
