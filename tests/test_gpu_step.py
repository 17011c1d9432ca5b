"""kvc_decode_step (append + attention in one call) on the GPU.

It must give exactly what kvc_append followed by kvc_decode_attn gives (same
split plan: bitwise equal caches, rotated query and output) and match the
oracle (bit-exact append, attention within tolerance), also at full size in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import GpuStep, bits, compare_out, oracle_append, oracle_decode, run_step, say, store_np

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_mha": W.WORKLOADS["tiny_mha"],
    "gqa_8b": W.WORKLOADS["gqa_8b"].replace(B=3, cached_lo=0, cached_hi=1100, T_max=1104),
    "mqa_ragged": W.WORKLOADS["mqa_ragged"].replace(B=5, cached_lo=100, cached_hi=700, T_max=704),
    "long_gqa": W.WORKLOADS["long_gqa"].replace(cached_lo=3000, cached_hi=3000, T_max=3008),
    "paged_gqa": W.WORKLOADS["paged_gqa"].replace(B=4, cached_lo=0, cached_hi=400),
    "gqa_d64": W.Workload("gqa_d64", 31, B=3, H_q=16, H_kv=4, d=64, dtype="bf16", cached_lo=10, cached_hi=500,
                          T_max=504),
    "mqa_d256": W.Workload("mqa_d256", 32, B=2, H_q=24, H_kv=1, d=256, dtype="bf16", cached_lo=10, cached_hi=500,
                           T_max=504),
    "valu_d32": W.Workload("valu_d32", 33, B=2, H_q=8, H_kv=2, d=32, dtype="bf16", cached_lo=10, cached_hi=300,
                           T_max=304),
    # the vector kernel with several head chunks per group: the new row is
    # stored by chunk 0 only and every chunk rotates its own queries
    "valu_f32_4chunks": W.Workload("valu_f32_4chunks", 34, B=2, H_q=64, H_kv=2, d=64, dtype="f32", cached_lo=10,
                                   cached_hi=300, T_max=304),
    "valu_bf16_8chunks": W.Workload("valu_bf16_8chunks", 35, B=2, H_q=64, H_kv=1, d=128, dtype="bf16",
                                    cached_lo=10, cached_hi=300, T_max=304),
}


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_step_equals_append_then_decode(name, style):
    x = W.draw(CASES[name])
    say(f"[step {name} {style}] lens={x.seq_lens.tolist()[:6]}")
    ref = GpuStep(x)
    # split 0 is the library plan, 64 leaves some waves without a tile, and one
    # split over the whole sequence gives every wave several tiles, so the new
    # token lands in a later tile of some wave
    for split in (0, 64, 1 << 20):
        k, v, q_rot, out = run_step(ref, split_tokens=split, rope_style=style)
        a = GpuStep(x)
        a.append(rope_style=style)
        out_a = a.decode(split_tokens=split)
        torch.cuda.synchronize()
        assert np.array_equal(bits(k), bits(a.k)), "K cache differs"
        assert np.array_equal(bits(v), bits(a.v)), "V cache differs"
        assert np.array_equal(bits(q_rot), bits(a.q)), "rotated q differs"
        if not np.array_equal(bits(out), bits(out_a)):
            bad = np.argwhere(bits(out).reshape(out.shape[0], out.shape[1], -1)
                              != bits(out_a).reshape(out.shape[0], out.shape[1], -1))
            say(f"  split {split}: output differs at (b, h) {sorted(set(map(tuple, bad[:, :2].tolist())))[:12]}")
        assert np.array_equal(bits(out), bits(out_a)), f"output differs (split {split})"
    # and against the oracle
    k2, v2, q2 = oracle_append(x, style)
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8))
    assert np.array_equal(bits(q_rot), np.ascontiguousarray(q2).view(np.uint8))
    compare_out(out, oracle_decode(x, k2, v2, q2), x.workload.dtype, f"step {name} {style}")


def test_step_out_of_range_positions_write_nothing():
    w = W.WORKLOADS["gqa_8b"].replace(B=3, cached_lo=50, cached_hi=50, T_max=64)
    x = W.draw(w)
    x.cached[:] = torch.tensor([10, 64, -1], dtype=torch.int32)     # 64 == T_max: outside the cache
    for b, c in enumerate(x.cached.tolist()):
        if c >= 0:
            x.k_cache[b, :, c:] = float("nan")
            x.v_cache[b, :, c:] = float("nan")
    say("[step] out-of-range positions")
    s = GpuStep(x)
    s.max_len = 64                       # the cache capacity; position 64 is outside it
    k0, v0 = bits(s.k), bits(s.v)
    k, v, q_rot, out = run_step(s)
    torch.cuda.synchronize()
    kb, vb = bits(k).reshape(3, -1), bits(v).reshape(3, -1)
    assert np.array_equal(kb[1:], k0.reshape(3, -1)[1:]) and np.array_equal(vb[1:], v0.reshape(3, -1)[1:])
    o = store_np(out, "bf16")
    assert np.all(o[1:] == 0)
    k2, v2, q2 = O.append_contiguous(store_np(x.k_cache[:1], "bf16"), store_np(x.v_cache[:1], "bf16"),
                                     x.cached.numpy()[:1], store_np(x.k_new[:1], "bf16"),
                                     store_np(x.v_new[:1], "bf16"), x.rope_cos.numpy(), x.rope_sin.numpy(),
                                     "bf16", q=store_np(x.q[:1], "bf16"))
    compare_out(out[:1], O.decode_attention(q2, k2, v2, [11], "bf16"), "bf16", "valid sequence")


def test_step_append_kernel_path_out_of_range_positions():
    """The step through the separate append kernel (float32 here): the query of
    a sequence whose slot is outside the cache reaches q_rot_out unrotated,
    as the documented append-on-a-copy would leave it; the others rotated."""
    w = W.WORKLOADS["tiny_mha"].replace(B=3, cached_lo=5, cached_hi=5, T_max=8)
    x = W.draw(w)
    x.cached[:] = torch.tensor([5, 8, -1], dtype=torch.int32)       # 8 == T_max: outside the cache
    say("[step tiny f32] out-of-range positions")
    s = GpuStep(x)
    s.max_len = 8
    k0, v0 = bits(s.k), bits(s.v)
    k, v, q_rot, out = run_step(s)
    torch.cuda.synchronize()
    qb = bits(q_rot).reshape(3, -1)
    assert np.array_equal(qb[1:], bits(x.q).reshape(3, -1)[1:]), "unrotated query expected"
    kb, vb = bits(k).reshape(3, -1), bits(v).reshape(3, -1)
    assert np.array_equal(kb[1:], k0.reshape(3, -1)[1:]) and np.array_equal(vb[1:], v0.reshape(3, -1)[1:])
    assert np.all(store_np(out, "f32")[1:] == 0)
    k2, v2, q2 = O.append_contiguous(store_np(x.k_cache[:1], "f32"), store_np(x.v_cache[:1], "f32"),
                                     x.cached.numpy()[:1], store_np(x.k_new[:1], "f32"),
                                     store_np(x.v_new[:1], "f32"), x.rope_cos.numpy(), x.rope_sin.numpy(),
                                     "f32", q=store_np(x.q[:1], "f32"))
    assert np.array_equal(qb[:1], np.ascontiguousarray(q2).view(np.uint8).reshape(1, -1)), "rotated q differs"
    compare_out(out[:1], O.decode_attention(q2, k2, v2, [6], "f32"), "f32", "valid sequence")


@pytest.mark.parametrize("name", ["gqa_8b", "mqa_ragged", "long_gqa", "paged_gqa", "tiny_mha"])
def test_step_full_size(name):
    """The benchmarked call (kvc_decode_step, default split plan) at full size,
    every output compared."""
    w = W.WORKLOADS[name]
    x = W.draw(w)
    say(f"[step {name} full] B={w.B} max_len={int(x.seq_lens.max())}")
    s = GpuStep(x)
    k, v, q_rot, out = run_step(s)
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs from the oracle"
    assert np.array_equal(bits(q_rot), np.ascontiguousarray(q2).view(np.uint8)), "rotated q differs"
    compare_out(out, oracle_decode(x, k2, v2, q2), w.dtype, f"step {name} full size")


@pytest.mark.parametrize("name", ["gqa_8b", "paged_gqa", "mqa_ragged"])
def test_prepared_step_equals_decode_step(name):
    """prepare_decode_step checks once and launches per call: each call gives
    bit for bit what decode_step gives on the buffers' contents at that time
    (a second call after the positions and the new token moved on)."""
    import mqa_decode_attention_amd as kvc
    x = W.draw(CASES[name])
    say(f"[prepared step {name}]")
    s = GpuStep(x)
    k, v = s.k.clone(), s.v.clone()
    q = x.q.to("cuda")
    pos = s.pos.clone()
    kn, vn = s.kn.clone(), s.vn.clone()
    out, q_rot = torch.empty_like(q), torch.empty_like(q)
    call = kvc.prepare_decode_step(q, k, v, pos, kn, vn, s.cos, s.sin, s.max_len + 1, block_table=s.tbl,
                                   q_rot_out=q_rot, out=out)
    k2, v2 = s.k.clone(), s.v.clone()
    for rnd in range(2):
        got = call()
        assert got[0] is out and got[1] is q_rot
        ref_out, ref_q = kvc.decode_step(q, k2, v2, pos, kn, vn, s.cos, s.sin, s.max_len + 1, block_table=s.tbl)
        torch.cuda.synchronize()
        assert np.array_equal(bits(k), bits(k2)) and np.array_equal(bits(v), bits(v2)), f"caches differ ({rnd})"
        assert np.array_equal(bits(q_rot), bits(ref_q)), f"rotated q differs ({rnd})"
        assert np.array_equal(bits(out), bits(ref_out)), f"output differs ({rnd})"
        # the next step: one position on, a new token
        pos += 1
        kn.copy_(torch.randn(kn.shape, generator=torch.Generator().manual_seed(rnd)).to(kn.dtype))
        vn.copy_(torch.randn(vn.shape, generator=torch.Generator().manual_seed(rnd + 9)).to(vn.dtype))


def test_last_split_takes_short_remainder():
    """With the library's split length over a contiguous cache, a sequence
    whose length exceeds a multiple of it by less than one kernel step (64
    tokens) has that remainder in its last split (4096 + 4097 for 8193
    tokens); by 64 or more, a split of its own.  Lengths on both sides of
    that edge, through the fused step and append + decode, against the
    oracle."""
    import mqa_decode_attention_amd as kvc
    # (drawn with every sequence full, then cut to the lengths wanted: slots
    # at and past each new length hold NaN again)
    w = W.WORKLOADS["gqa_8b"].replace(B=4, cached_lo=1099, cached_hi=1099, T_max=1104)
    x = W.draw(w)
    M = 1100
    ts = kvc.split_tokens(torch.bfloat16, w.B, w.H_q, w.H_kv, w.d, M)
    q = (M - 64) // ts
    lens = [q * ts + 1, q * ts + 63, q * ts + 64, M]
    assert len(set(lens)) == 4 and max(lens) == M and all(L % ts for L in lens[:3])
    x.cached[:] = torch.tensor([L - 1 for L in lens], dtype=torch.int32)
    x.seq_lens[:] = torch.tensor(lens, dtype=torch.int32)
    for b, c in enumerate(x.cached.tolist()):
        x.k_cache[b, :, c:] = float("nan")
        x.v_cache[b, :, c:] = float("nan")
    say(f"[remainder] split {ts}, lengths {lens}")
    s = GpuStep(x)
    assert s.max_len == M
    k, v, q_rot, out = run_step(s)
    a = GpuStep(x)
    a.append()
    out_a = a.decode()
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), bits(a.k)) and np.array_equal(bits(v), bits(a.v))
    assert np.array_equal(bits(out), bits(out_a)), "step differs from append + decode"
    k2, v2, q2 = oracle_append(x)
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8))
    compare_out(out, oracle_decode(x, k2, v2, q2), w.dtype, "remainder in the last split")
