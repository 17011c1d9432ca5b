"""Seeded input generators: determinism, layout, poison placement (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W


def _small(name):
    w = W.WORKLOADS[name]
    if name == "tiny_mha":
        return w
    if w.paged:
        return w.replace(B=3, cached_lo=20, cached_hi=70)
    lo = min(w.cached_lo, 40)
    hi = min(w.cached_hi, 90) if w.cached_hi != w.cached_lo else lo
    return w.replace(B=min(w.B, 3), cached_lo=lo, cached_hi=hi, T_max=hi + 8)


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_shapes_and_determinism(name):
    w = _small(name)
    a, b = W.draw(w), W.draw(w)
    for f in ("cached", "k_cache", "v_cache", "q", "k_new", "v_new", "rope_cos", "rope_sin"):
        x, y = getattr(a, f), getattr(b, f)
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y), f
    want = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    assert a.q.dtype == want and a.k_cache.dtype == want
    tok = (w.new_tokens,) if w.new_tokens > 1 else ()
    assert a.q.shape == (w.B,) + tok + (w.H_q, w.d) and a.k_new.shape == (w.B,) + tok + (w.H_kv, w.d)
    assert a.rope_cos.shape == (w.table_rows, w.d // 2)
    assert int(a.cached.min()) >= w.cached_lo and int(a.cached.max()) <= w.cached_hi
    if w.paged:
        nblk = [-(-int(L) // w.block_size) for L in a.seq_lens]
        assert a.k_cache.shape == (sum(nblk), w.H_kv, w.block_size, w.d)
        used = torch.cat([a.block_table[b, :n] for b, n in enumerate(nblk)])
        assert sorted(used.tolist()) == list(range(sum(nblk)))      # a permutation
        for b, n in enumerate(nblk):
            assert torch.all(a.block_table[b, n:] == -1)
    else:
        assert a.k_cache.shape == (w.B, w.H_kv, w.T_max, w.d)


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_poison_exactly_past_cached_length(name):
    w = _small(name)
    x = W.draw(w)
    for b, c in enumerate(x.cached.tolist()):
        if w.paged:
            bs = w.block_size
            for p in range(0, -(-(c + w.new_tokens) // bs) * bs):
                blk = int(x.block_table[b, p // bs])
                row = x.k_cache[blk, :, p % bs].float()
                assert bool(torch.isnan(row).all()) == (p >= c)
        else:
            kb = x.k_cache[b].float()
            assert torch.isfinite(kb[:, :c]).all() and torch.isnan(kb[:, c:]).all()
            assert torch.isnan(x.v_cache[b].float()[:, c:]).all()


def test_different_seeds_differ_and_ragged_lengths_spread():
    w = W.WORKLOADS["mqa_ragged"].replace(T_max=4104)
    x = W.draw(w.replace(B=64, cached_lo=512, cached_hi=4096, T_max=4104))
    lens = x.cached.numpy()
    assert lens.min() >= 512 and lens.max() <= 4096 and len(np.unique(lens)) > 32
    y = W.draw(w.replace(seed=99, B=2, cached_lo=5, cached_hi=9, T_max=16))
    z = W.draw(w.replace(B=2, cached_lo=5, cached_hi=9, T_max=16))
    assert not torch.equal(y.q.float(), z.q.float())


def test_full_size_table_shapes():
    assert W.WORKLOADS["paged_gqa"].max_blocks_per_seq == 1025
    assert W.WORKLOADS["gqa_8b"].G == 4 and W.WORKLOADS["long_gqa"].G == 8
    assert W.WORKLOADS["mqa_ragged"].G == 32 and W.WORKLOADS["tiny_mha"].G == 1
