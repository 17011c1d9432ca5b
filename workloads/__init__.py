"""Seeded synthetic inputs for one decode step of grouped-query attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no attention, no rounding rules of its own:
casting to bfloat16 is torch's round-to-nearest-even). Both the CPU oracle's
tests and the GPU path's tests/benchmark take their inputs from here, and from
nowhere else, so that the two sides see byte-identical data.

Workloads (the shapes of the pages' examples, synthetic values N(0, 1)):

* ``tiny_mha``   batch 1, 4 query / 4 KV heads, head dim 16, 5 cached tokens
                 (+1 appended), fp32, RoPE base 10000.
* ``gqa_8b``     batch 16, 32 query / 8 KV heads (G = 4), head dim 128, 8192
                 cached tokens per sequence, bf16, contiguous cache.  The layer
                 shape of an 8B model with 8 KV groups for 32 heads.
* ``mqa_ragged`` batch 64, 32 query heads sharing 1 KV head, head dim 128,
                 cached lengths uniform in [512, 4096], bf16.
* ``long_gqa``   batch 1, 64 query / 8 KV heads (G = 8), head dim 128, 131072
                 cached tokens, bf16.
* ``paged_gqa``  batch 32, 32 / 8 heads, head dim 128, block size 16, cached
                 lengths uniform in [1024, 16384]; the blocks of all sequences
                 sit in one shared pool in a seeded random order.
* ``spec_gqa``   gqa_8b's shape with 6 new tokens per sequence: the target
                 model checking gamma = 5 drafted tokens in one pass, the
                 worked example of speculative decoding in "Arsitektur
                 Inferensi LLM" (tveniu.com), section 7.

A workload with ``new_tokens`` = n > 1 draws q [B, n, H_q, d] and k_new,
v_new [B, n, H_kv, d] (token-major); the cache then has room for, and NaN in,
the n slots the append fills.

Draw order (one ``torch.Generator`` seeded with the workload's seed):
cached lengths -> block permutation (paged only) -> K cache -> V cache -> q ->
k_new -> v_new.  Values are drawn as float32 N(0, 1) and cast to the storage
dtype.  Every cache slot at or past a sequence's cached length (including the
slot the append will fill) holds NaN, so a read of an unwritten slot shows up.

The RoPE cos/sin table is an input of the append (the pages do not give the
rotation frequencies): row p, column i holds cos/sin(p * base^(-2i/d)),
evaluated in float64 and rounded once to float32.

Quantized cache (``draw_quantized``): the same workload's layout with uint8
codes in place of the K and V values and a float32 (step, zero point) pair per
cached vector, drawn directly (this module does no quantizing), with the
statistics such a cache of N(0, 1) vectors has: steps uniform in
[0.015, 0.03) (the range (max - min) / 255 takes for vectors of a few hundred
elements), zero points integers uniform in [100, 155], and codes a normal
sample around the zero point with spread 1 / step, rounded to an integer and
kept in [0, 255] - so each vector reads back as roughly N(0, 1) values.  From a
second generator seeded with seed + 7919, in the order K pairs -> V pairs ->
K codes -> V codes, so the unquantized draws stay unchanged.  Slots at or past
a sequence's cached length hold code 0 and NaN pairs.

FP8 cache (``draw_fp8``): the same layout with one-byte E4M3 or E5M2 codes and
float32 (scale, 0) pairs, codes drawn as torch's float8 casts of N(0, 1) /
scale (the casts are torch's, as the bfloat16 casts above), scales uniform in
[2.5, 3.5) / 448 for E4M3 and 1 for E5M2 (see ``draw_fp8``).

Latent cache (``MLA_WORKLOADS``, ``draw_mla``): the cache layout of the
MultiHeadLatentAttention listing in "KV Cache 최적화 심층 분석" (youngju.dev),
one row [c_kv | k_rope] of d_latent + rope_dim values per token, [B, T_max,
d_latent + rope_dim].  Values N(0, 1) as above (NaN at and past each cached
length); q [B, n_heads, d_k] N(0, 1); the new token's c_kv [B, d_latent] and
k_rope [B, rope_dim] N(0, 1); the up-projections W_uk, W_uv [n_heads * d_k,
d_latent] and their biases [n_heads * d_k] drawn as torch's nn.Linear
initialises them, uniform in +-1/sqrt(d_latent).  Draw order: cached lengths
-> cache -> q -> c_kv -> k_rope -> W_uk -> b_uk -> W_uv -> b_uv.  There are no
trained weights anywhere: these only give the products realistic scales.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "DecodeInputs", "QuantCache", "draw", "draw_quantized", "draw_fp8",
           "rotation_table", "MlaWorkload", "MLA_WORKLOADS", "MlaInputs", "draw_mla"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H_q: int
    H_kv: int
    d: int
    dtype: str                 # "f32" or "bf16": storage dtype of q, K, V, out
    cached_lo: int             # cached tokens per sequence before the step,
    cached_hi: int             # uniform integers in [lo, hi] (equal => fixed)
    layout: str = "contiguous"  # or "paged"
    T_max: int = 0             # contiguous capacity (tokens per (b, kv head))
    block_size: int = 16       # paged only
    new_tokens: int = 1        # tokens appended (and queries attending) per sequence
    rope_base: float = 10000.0

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def paged(self) -> bool:
        return self.layout == "paged"

    @property
    def max_attended(self) -> int:
        return self.cached_hi + self.new_tokens

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_attended // self.block_size)

    @property
    def table_rows(self) -> int:
        """Positions the rotation table covers (every slot a sequence can use)."""
        if self.paged:
            return self.max_blocks_per_seq * self.block_size
        return self.T_max

    def replace(self, **kw) -> "Workload":
        """Same structure at another size (for oracle-sized parity cases)."""
        w = dataclasses.replace(self, **kw)
        if not w.paged and w.T_max < w.cached_hi + w.new_tokens:
            w = dataclasses.replace(w, T_max=_round_up(w.cached_hi + w.new_tokens, 8))
        return w


def _round_up(x: int, m: int) -> int:
    return -(-x // m) * m


WORKLOADS = {
    "tiny_mha": Workload("tiny_mha", 0, B=1, H_q=4, H_kv=4, d=16, dtype="f32",
                         cached_lo=5, cached_hi=5, T_max=8),
    "gqa_8b": Workload("gqa_8b", 1, B=16, H_q=32, H_kv=8, d=128, dtype="bf16",
                       cached_lo=8192, cached_hi=8192, T_max=8200),
    "mqa_ragged": Workload("mqa_ragged", 2, B=64, H_q=32, H_kv=1, d=128, dtype="bf16",
                           cached_lo=512, cached_hi=4096, T_max=4104),
    "long_gqa": Workload("long_gqa", 3, B=1, H_q=64, H_kv=8, d=128, dtype="bf16",
                         cached_lo=131072, cached_hi=131072, T_max=131080),
    "paged_gqa": Workload("paged_gqa", 4, B=32, H_q=32, H_kv=8, d=128, dtype="bf16",
                          cached_lo=1024, cached_hi=16384, layout="paged", block_size=16),
    "spec_gqa": Workload("spec_gqa", 5, B=16, H_q=32, H_kv=8, d=128, dtype="bf16",
                         cached_lo=8192, cached_hi=8192, T_max=8200, new_tokens=6),
}


@dataclasses.dataclass
class DecodeInputs:
    """One decode step's inputs, on the CPU, in storage dtype.

    cached      int32 [B]   tokens in the cache before the step (= append slot)
    k_cache     [B, H_kv, T_max, d]   contiguous layout, or
                [N_blocks, H_kv, block_size, d]   paged pool
    v_cache     same shape as k_cache
    block_table int32 [B, max_blocks_per_seq] (paged; -1 = unused) or None
    q           [B, H_q, d]   raw (not yet rotated) query of the new token
                ([B, n, H_q, d] for n = new_tokens > 1)
    k_new, v_new [B, H_kv, d] raw key and value of the new token ([B, n, H_kv, d])
    rope_cos, rope_sin  float32 [table_rows, d // 2]
    """
    workload: Workload
    cached: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor]
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    rope_cos: torch.Tensor
    rope_sin: torch.Tensor

    @property
    def seq_lens(self) -> torch.Tensor:
        """Length after the append (cached + new tokens)."""
        return self.cached + self.workload.new_tokens


def _storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(f"unknown dtype {dtype!r}")


def rotation_table(rows: int, d: int, base: float = 10000.0):
    """cos/sin of p * base^(-2i/d) for p < rows, i < d/2; float64 -> float32 once."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / d)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


def draw(w: Workload) -> DecodeInputs:
    """Draw the workload's inputs from its seed (deterministic, CPU only)."""
    g = torch.Generator().manual_seed(w.seed)
    if w.cached_lo == w.cached_hi:
        cached = torch.full((w.B,), w.cached_lo, dtype=torch.int32)
    else:
        cached = torch.randint(w.cached_lo, w.cached_hi + 1, (w.B,), generator=g,
                               dtype=torch.int64).to(torch.int32)
    n_new = w.new_tokens
    lens = (cached + n_new).tolist()

    block_table = None
    if w.paged:
        bs = w.block_size
        nblk = [-(-L // bs) for L in lens]
        total = sum(nblk)
        perm = torch.randperm(total, generator=g).to(torch.int32)
        block_table = torch.full((w.B, w.max_blocks_per_seq), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(nblk):
            block_table[b, :n] = perm[off:off + n]
            off += n
        shape = (total, w.H_kv, bs, w.d)
    else:
        assert w.T_max >= w.cached_hi + n_new, "contiguous capacity must hold the cached and new tokens"
        shape = (w.B, w.H_kv, w.T_max, w.d)

    k_cache = torch.randn(shape, generator=g, dtype=torch.float32)
    v_cache = torch.randn(shape, generator=g, dtype=torch.float32)
    tok = (n_new,) if n_new > 1 else ()
    q = torch.randn((w.B,) + tok + (w.H_q, w.d), generator=g, dtype=torch.float32)
    k_new = torch.randn((w.B,) + tok + (w.H_kv, w.d), generator=g, dtype=torch.float32)
    v_new = torch.randn((w.B,) + tok + (w.H_kv, w.d), generator=g, dtype=torch.float32)

    k_cache = _storage(k_cache, w.dtype)
    v_cache = _storage(v_cache, w.dtype)
    nan = float("nan")
    for b, c in enumerate(cached.tolist()):
        if w.paged:
            bs = w.block_size
            for p in range(c, -(-lens[b] // bs) * bs):
                blk = int(block_table[b, p // bs])
                k_cache[blk, :, p % bs, :] = nan
                v_cache[blk, :, p % bs, :] = nan
        else:
            k_cache[b, :, c:, :] = nan
            v_cache[b, :, c:, :] = nan

    cos, sin = rotation_table(w.table_rows, w.d, w.rope_base)
    return DecodeInputs(w, cached, k_cache, v_cache, block_table,
                        _storage(q, w.dtype), _storage(k_new, w.dtype),
                        _storage(v_new, w.dtype), cos, sin)


@dataclasses.dataclass
class QuantCache:
    """A quantized cache of a workload's layout, on the CPU.

    k_codes, v_codes  uint8 [B, H_kv, T_max, d] or [N_blocks, H_kv, block_size, d]
    k_sz, v_sz        float32 [..., 2]: (step, zero point) of each cached vector
    """
    k_codes: torch.Tensor
    k_sz: torch.Tensor
    v_codes: torch.Tensor
    v_sz: torch.Tensor


def draw_quantized(x: DecodeInputs) -> QuantCache:
    """Draw a quantized cache in the layout of x (same lengths and block table)."""
    w = x.workload
    g = torch.Generator().manual_seed(w.seed + 7919)
    shape = tuple(x.k_cache.shape)
    lead = shape[:-1]
    pairs = []
    for _ in range(2):
        step = 0.015 + 0.015 * torch.rand(lead, generator=g, dtype=torch.float32)
        zp = torch.randint(100, 156, lead, generator=g, dtype=torch.int64).to(torch.float32)
        pairs.append(torch.stack([step, zp], dim=-1).contiguous())
    k_sz, v_sz = pairs
    codes = []
    for sz in (k_sz, v_sz):
        c = torch.randn(shape, generator=g, dtype=torch.float32) / sz[..., :1] + sz[..., 1:]
        codes.append(torch.round(c).clamp(0, 255).to(torch.uint8).contiguous())
    k_codes, v_codes = codes
    nan = float("nan")
    lens = (x.cached + 1).tolist()
    for b, c in enumerate(x.cached.tolist()):
        if w.paged:
            bs = w.block_size
            for pos in range(c, -(-lens[b] // bs) * bs):
                blk = int(x.block_table[b, pos // bs])
                for t in (k_codes, v_codes):
                    t[blk, :, pos % bs, :] = 0
                for t in (k_sz, v_sz):
                    t[blk, :, pos % bs, :] = nan
        else:
            for t in (k_codes, v_codes):
                t[b, :, c:, :] = 0
            for t in (k_sz, v_sz):
                t[b, :, c:, :] = nan
    return QuantCache(k_codes, k_sz, v_codes, v_sz)


def draw_fp8(x: DecodeInputs, fmt: str) -> QuantCache:
    """Draw an FP8 cache (fmt "e4m3" or "e5m2") in the layout of x: uint8 codes
    and float32 (scale, 0) pairs per cached vector.

    E4M3: scales uniform in [2.5, 3.5) / 448 (the largest magnitude of a few
    hundred N(0, 1) values over the format's largest value) and codes torch's
    float8_e4m3fn cast of N(0, 1) / scale, kept within +-448; E5M2: scale 1
    and torch's float8_e5m2 cast of N(0, 1).  Either reads back as roughly
    N(0, 1) values.  From a generator seeded with seed + 7919 + 1 (E4M3) or
    + 2 (E5M2), in the order K scales -> V scales -> K codes -> V codes.  Slots
    at or past a sequence's cached length hold code 0 and NaN pairs.
    """
    w = x.workload
    g = torch.Generator().manual_seed(w.seed + 7919 + (1 if fmt == "e4m3" else 2))
    shape = tuple(x.k_cache.shape)
    lead = shape[:-1]
    cast = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    pairs = []
    for _ in range(2):
        if fmt == "e4m3":
            scale = (2.5 + torch.rand(lead, generator=g, dtype=torch.float32)) / 448.0
        else:
            scale = torch.ones(lead, dtype=torch.float32)
        pairs.append(torch.stack([scale, torch.zeros(lead)], dim=-1).contiguous())
    k_sz, v_sz = pairs
    codes = []
    for sz in (k_sz, v_sz):
        c = torch.randn(shape, generator=g, dtype=torch.float32) / sz[..., :1]
        if fmt == "e4m3":
            c = c.clamp(-448.0, 448.0)
        codes.append(c.to(cast).view(torch.uint8).contiguous())
    k_codes, v_codes = codes
    nan = float("nan")
    lens = (x.cached + 1).tolist()
    for b, c in enumerate(x.cached.tolist()):
        if w.paged:
            bs = w.block_size
            for pos in range(c, -(-lens[b] // bs) * bs):
                blk = int(x.block_table[b, pos // bs])
                for t in (k_codes, v_codes):
                    t[blk, :, pos % bs, :] = 0
                for t in (k_sz, v_sz):
                    t[blk, :, pos % bs, :] = nan
        else:
            for t in (k_codes, v_codes):
                t[b, :, c:, :] = 0
            for t in (k_sz, v_sz):
                t[b, :, c:, :] = nan
    return QuantCache(k_codes, k_sz, v_codes, v_sz)


@dataclasses.dataclass(frozen=True)
class MlaWorkload:
    """A decode step over a latent cache: n_heads query heads of width d_k,
    each token cached as one row of d_latent + rope_dim values."""
    name: str
    seed: int
    B: int
    H: int                     # query heads (n_heads)
    d_k: int                   # per-head width of q and of the output
    d_latent: int
    rope_dim: int
    dtype: str                 # "bf16": storage dtype of the cache, q and weights
    cached_lo: int
    cached_hi: int
    T_max: int = 0

    @property
    def row(self) -> int:
        return self.d_latent + self.rope_dim

    @property
    def max_attended(self) -> int:
        return self.cached_hi + 1

    def replace(self, **kw) -> "MlaWorkload":
        w = dataclasses.replace(self, **kw)
        if w.T_max < w.cached_hi + 1:
            w = dataclasses.replace(w, T_max=_round_up(w.cached_hi + 1, 8))
        return w


MLA_WORKLOADS = {
    # the 8B-class layer of gqa_8b (32 heads of 128, batch 16, 8192 cached
    # tokens) with a 512-wide latent and the listing's default rope_dim 64
    "mla_latent": MlaWorkload("mla_latent", 6, B=16, H=32, d_k=128, d_latent=512, rope_dim=64, dtype="bf16",
                              cached_lo=8192, cached_hi=8192, T_max=8200),
}


@dataclasses.dataclass
class MlaInputs:
    """One latent-cache decode step's inputs, on the CPU, in storage dtype.

    cached   int32 [B]                tokens cached before the step (= append slot)
    cache    [B, T_max, d_latent + rope_dim]
    q        [B, H, d_k]
    c_kv_new [B, d_latent], k_rope_new [B, rope_dim]
    w_uk, w_uv [H * d_k, d_latent];  b_uk, b_uv [H * d_k]
    """
    workload: MlaWorkload
    cached: torch.Tensor
    cache: torch.Tensor
    q: torch.Tensor
    c_kv_new: torch.Tensor
    k_rope_new: torch.Tensor
    w_uk: torch.Tensor
    b_uk: torch.Tensor
    w_uv: torch.Tensor
    b_uv: torch.Tensor

    @property
    def seq_lens(self) -> torch.Tensor:
        return self.cached + 1


def draw_mla(w: MlaWorkload) -> MlaInputs:
    """Draw a latent-cache workload's inputs from its seed (deterministic, CPU only)."""
    g = torch.Generator().manual_seed(w.seed)
    if w.cached_lo == w.cached_hi:
        cached = torch.full((w.B,), w.cached_lo, dtype=torch.int32)
    else:
        cached = torch.randint(w.cached_lo, w.cached_hi + 1, (w.B,), generator=g,
                               dtype=torch.int64).to(torch.int32)
    assert w.T_max >= w.cached_hi + 1, "the cache must hold the cached and the new token"
    cache = torch.randn((w.B, w.T_max, w.row), generator=g, dtype=torch.float32)
    q = torch.randn((w.B, w.H, w.d_k), generator=g, dtype=torch.float32)
    c_kv = torch.randn((w.B, w.d_latent), generator=g, dtype=torch.float32)
    k_rope = torch.randn((w.B, w.rope_dim), generator=g, dtype=torch.float32)
    bound = 1.0 / math.sqrt(w.d_latent)
    uni = lambda *shape: (torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0) * bound
    w_uk, b_uk = uni(w.H * w.d_k, w.d_latent), uni(w.H * w.d_k)
    w_uv, b_uv = uni(w.H * w.d_k, w.d_latent), uni(w.H * w.d_k)
    cache = _storage(cache, w.dtype)
    for b, c in enumerate(cached.tolist()):
        cache[b, c:, :] = float("nan")
    st = lambda t: _storage(t, w.dtype)
    return MlaInputs(w, cached, cache, st(q), st(c_kv), st(k_rope), st(w_uk), st(b_uk), st(w_uv), st(b_uv))
