"""GPU parity of multi-token decode (n new tokens per sequence, each query
causal over the cache and the new tokens up to itself) with its oracle,
through the C ABI.

* kvc_append_multi must write the oracle's caches and rotated queries bit for
  bit (contiguous and paged).
* kvc_decode_attn_multi must match the oracle within the bf16 bar for query
  row counts G * n from 4 to 64 (one or two 16-row head blocks, one or two
  chunks of 32 rows), head_dim 64 / 128 / 256, every paged mode, with and
  without a window, for several splits; with n = 1 it must equal the
  single-token kvc_decode_attn bit for bit.
* spec_gqa at full size (16 sequences x 8192 cached + 6 new tokens), every
  output, in the library's launch plan.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import oracle as O
import oracle.kvc_multi_oracle as MO
import workloads as W
from gpu_helpers import bits, compare_out, say, store_np

pytestmark = pytest.mark.gpu

G8 = W.WORKLOADS["gqa_8b"]
PG = W.WORKLOADS["paged_gqa"]
CASES = {
    # name: (workload, window)
    "g4_n6": (G8.replace(B=3, cached_lo=300, cached_hi=1100, new_tokens=6), 0),       # 24 rows
    "g4_n2": (G8.replace(B=2, cached_lo=100, cached_hi=600, new_tokens=2), 0),        # 8 rows
    "g4_n8_w": (G8.replace(B=3, cached_lo=200, cached_hi=700, new_tokens=8), 150),    # 32 rows, window
    "mha_n5": (G8.replace(B=2, H_q=8, H_kv=8, cached_lo=50, cached_hi=400, new_tokens=5), 0),
    "g8_n6": (G8.replace(B=2, H_q=64, cached_lo=100, cached_hi=500, new_tokens=6), 0),  # 48 rows: 2 chunks
    "mqa_n2": (G8.replace(B=3, H_kv=1, cached_lo=100, cached_hi=400, new_tokens=2), 0),  # 64 rows
    "g4_d64_n3": (G8.replace(B=2, d=64, cached_lo=90, cached_hi=300, new_tokens=3), 0),
    "g4_d256_n4": (G8.replace(B=2, d=256, cached_lo=90, cached_hi=300, new_tokens=4), 40),
    "paged_n6": (PG.replace(B=4, cached_lo=20, cached_hi=400, new_tokens=6), 0),       # staged tiles
    "paged_n4_w": (PG.replace(B=3, cached_lo=30, cached_hi=300, new_tokens=4), 37),
    "paged_d256_n3": (PG.replace(B=3, d=256, H_q=16, H_kv=4, cached_lo=40, cached_hi=300, new_tokens=3), 0),
    "paged_bs8_n5": (PG.replace(B=3, block_size=8, cached_lo=30, cached_hi=300, new_tokens=5), 0),
}


class MultiStep:
    def __init__(self, x: W.DecodeInputs, device="cuda"):
        w = x.workload
        self.x = x
        self.k, self.v = x.k_cache.to(device), x.v_cache.to(device)
        self.q = x.q.to(device).clone()
        self.kn, self.vn = x.k_new.to(device), x.v_new.to(device)
        self.pos, self.lens = x.cached.to(device), x.seq_lens.to(device)
        self.cos, self.sin = x.rope_cos.to(device), x.rope_sin.to(device)
        self.tbl = x.block_table.to(device) if w.paged else None
        self.max_len = int(x.seq_lens.max())

    def append(self):
        kvc.append_multi(self.k, self.v, self.pos, self.kn, self.vn, self.cos, self.sin, q=self.q,
                         block_table=self.tbl)

    def decode(self, window=0, split=0):
        return kvc.decode_attn_multi(self.q, self.k, self.v, self.lens, self.max_len, window,
                                     block_table=self.tbl, split_tokens=split)


def oracle_append_multi(x: W.DecodeInputs):
    w = x.workload
    dt = w.dtype
    kc, vc = store_np(x.k_cache, dt), store_np(x.v_cache, dt)
    q, kn, vn = store_np(x.q, dt), store_np(x.k_new, dt), store_np(x.v_new, dt)
    cos, sin = x.rope_cos.numpy(), x.rope_sin.numpy()
    if w.paged:
        return MO.append_multi_paged(kc, vc, x.block_table.numpy(), w.block_size, x.cached.numpy(), kn, vn, cos,
                                     sin, dt, q=q)
    return MO.append_multi(kc, vc, x.cached.numpy(), kn, vn, cos, sin, dt, q=q)


def oracle_decode_multi(x, k2, v2, q2, window):
    w = x.workload
    lens = x.seq_lens.numpy()
    if w.paged:
        return MO.decode_attention_multi_paged(q2, k2, v2, x.block_table.numpy(), w.block_size, lens, w.dtype,
                                               window)
    return MO.decode_attention_multi(q2, k2, v2, lens, w.dtype, window)


def _append_and_check(step: MultiStep, x):
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append_multi(x)
    assert np.array_equal(bits(step.k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(step.v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs from the oracle"
    assert np.array_equal(store_np(step.q, x.workload.dtype).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8)), \
        "rotated queries differ from the oracle"
    return k2, v2, q2


@pytest.mark.parametrize("name", sorted(CASES))
def test_multi_matches_oracle(name):
    wl, window = CASES[name]
    x = W.draw(wl)
    say(f"[multi {name}] G={wl.G} n={wl.new_tokens} d={wl.d} W={window} lens={x.seq_lens.tolist()[:6]}")
    step = MultiStep(x)
    k2, v2, q2 = _append_and_check(step, x)
    ref = oracle_decode_multi(x, k2, v2, q2, window)
    for split in (0, 64, 1 << 20):
        out = step.decode(window, split)
        torch.cuda.synchronize()
        compare_out(out, ref, "bf16", f"{name} split={split}")


def test_multi_single_token_equals_decode():
    """n = 1 through kvc_decode_attn_multi (the multi-token kernel: per-row
    causal bounds, row map, output rows) == kvc_decode_attn bit for bit: the
    same tiles in the same order."""
    x = W.draw(G8.replace(B=3, cached_lo=300, cached_hi=900))
    dev = "cuda"
    k, v = x.k_cache.to(dev), x.v_cache.to(dev)
    q = x.q.to(dev).clone()
    kvc.append(k, v, x.cached.to(dev), x.k_new.to(dev), x.v_new.to(dev), x.rope_cos.to(dev), x.rope_sin.to(dev), q=q)
    lens = x.seq_lens.to(dev)
    L = int(x.seq_lens.max())
    for split in (0, 64):
        one = kvc.decode_attn(q, k, v, lens, L, split_tokens=split)
        multi = kvc.decode_attn_multi(q[:, None].contiguous(), k, v, lens, L, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16), multi[:, 0].view(torch.int16)), f"split {split}"


def test_multi_full_size():
    """spec_gqa: 16 sequences x (8192 cached + 6 new), the library's plan, the
    append bit for bit and every output compared."""
    w = W.WORKLOADS["spec_gqa"]
    x = W.draw(w)
    say(f"[multi full spec_gqa] n={w.new_tokens}")
    step = MultiStep(x)
    k2, v2, q2 = _append_and_check(step, x)
    out = step.decode()
    torch.cuda.synchronize()
    compare_out(out, oracle_decode_multi(x, k2, v2, q2, 0), w.dtype, "spec_gqa full size")
