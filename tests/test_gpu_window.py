"""GPU parity of sliding-window decode with its oracle, through the C ABI.

* kvc_decode_attn_window over a full cache (contiguous; paged through each of
  the paged kernels' modes: 16-row staged tiles at d = 128, per-group tables at
  d = 256, per-row tables at block size 8; float32 through the vector kernel)
  must match the oracle's attention over tokens [max(0, L - W), L) within the
  bf16 / fp32 bars, for windows from 1 token to past the whole sequence and
  for several splits.  Every token before a sequence's window is NaN (and the
  table entries of blocks wholly before it are -1), so reading any of them
  would show.
* kvc_append_ring must write the oracle's ring bit for bit, and the ring
  decode must match the oracle's decode over the ring's slots.
* kvc_decode_step_window must equal the oracle's append + windowed decode, and
  equal kvc_append + kvc_decode_attn_window bit for bit (full cache and ring).
* At the gqa_8b workload's full size with Mistral's 4096-token window, every
  output, in the launch configuration of the library's plan.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import oracle as O
import oracle.kvc_window_oracle as WO
import workloads as W
from gpu_helpers import GpuStep, bits, compare_out, oracle_append, say, store_np

pytestmark = pytest.mark.gpu

SMALL = {
    "gqa_8b": W.WORKLOADS["gqa_8b"].replace(B=3, cached_lo=300, cached_hi=1100, T_max=1104),
    "mqa_ragged": W.WORKLOADS["mqa_ragged"].replace(B=5, cached_lo=100, cached_hi=700, T_max=704),
    "paged_gqa": W.WORKLOADS["paged_gqa"].replace(B=4, cached_lo=20, cached_hi=400),
    "paged_d256": W.WORKLOADS["paged_gqa"].replace(B=3, d=256, H_q=16, H_kv=4, cached_lo=50, cached_hi=300),
    "paged_bs8": W.WORKLOADS["paged_gqa"].replace(B=3, block_size=8, cached_lo=30, cached_hi=300),
    "gqa_f32": W.WORKLOADS["gqa_8b"].replace(B=2, d=64, dtype="f32", cached_lo=200, cached_hi=500),
}
WINDOWS = (1, 16, 37, 100, 257, 5000)


def poison_before_window(x: W.DecodeInputs, window: int) -> None:
    """NaN every cached token before each sequence's window (after this step's
    append, L = cached + 1); paged: also -1 the table entries of blocks that
    lie wholly before it."""
    w = x.workload
    nan = float("nan")
    for b, L in enumerate(x.seq_lens.tolist()):
        lo = WO.window_start(L, window)
        if w.paged:
            bs = w.block_size
            for t in range(lo):
                blk = int(x.block_table[b, t // bs])
                x.k_cache[blk, :, t % bs] = nan
                x.v_cache[blk, :, t % bs] = nan
            x.block_table[b, :lo // bs] = -1
        else:
            x.k_cache[b, :, :lo] = nan
            x.v_cache[b, :, :lo] = nan


def oracle_window(x: W.DecodeInputs, k2, v2, q2, window: int):
    w = x.workload
    lens = x.seq_lens.numpy()
    if w.paged:
        return WO.decode_attention_window_paged(q2, k2, v2, x.block_table.numpy(), w.block_size, lens, window,
                                                w.dtype)
    return WO.decode_attention_window(q2, k2, v2, lens, window, w.dtype)


def _append_and_check(step: GpuStep, x):
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    assert np.array_equal(bits(step.k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(step.v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs from the oracle"
    return k2, v2, q2


def _decode_window(step: GpuStep, window, split=0):
    return kvc.decode_attn_window(step.q, step.k, step.v, step.lens, step.max_len, window,
                                  block_table=step.tbl, split_tokens=split)


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("name", sorted(SMALL))
def test_window_matches_oracle(name, window):
    x = W.draw(SMALL[name])
    w = x.workload
    poison_before_window(x, window)
    say(f"[window {name} W={window}] d={w.d} lens={x.seq_lens.tolist()[:6]}")
    step = GpuStep(x)
    k2, v2, q2 = _append_and_check(step, x)
    ref = oracle_window(x, k2, v2, q2, window)
    splits = (0, 64, 1 << 20) if w.paged else (0, 64, 100, 1 << 20)
    for split in splits:
        out = _decode_window(step, window, split)
        torch.cuda.synchronize()
        compare_out(out, ref, w.dtype, f"{name} W={window} split={split}")


def test_window_edge_lengths():
    """L = 1, windows ending exactly on a tile / block boundary, L = 0."""
    base = W.WORKLOADS["paged_gqa"].replace(B=5, cached_lo=100, cached_hi=100)
    for layout in ("contiguous", "paged"):
        wl = base if layout == "paged" else base.replace(layout="contiguous", T_max=0)
        x = W.draw(wl)
        x.cached[:] = torch.tensor([0, 15, 16, 63, 100], dtype=torch.int32)
        for window in (16, 48):
            xs = W.draw(wl)
            xs.cached[:] = x.cached
            # re-poison for the new lengths: past L and before the window
            for b, c in enumerate(xs.cached.tolist()):
                if xs.workload.paged:
                    for t in range(c, xs.block_table.shape[1] * xs.workload.block_size):
                        blk = int(xs.block_table[b, t // xs.workload.block_size])
                        if blk >= 0:
                            xs.k_cache[blk, :, t % xs.workload.block_size] = float("nan")
                            xs.v_cache[blk, :, t % xs.workload.block_size] = float("nan")
                else:
                    xs.k_cache[b, :, c:] = float("nan")
                    xs.v_cache[b, :, c:] = float("nan")
            poison_before_window(xs, window)
            say(f"[window edge {layout} W={window}] lens={xs.seq_lens.tolist()}")
            step = GpuStep(xs)
            k2, v2, q2 = _append_and_check(step, xs)
            ref = oracle_window(xs, k2, v2, q2, window)
            for split in (0, 16, 1 << 20):
                compare_out(_decode_window(step, window, split), ref, "bf16", f"{layout} W={window} split={split}")
            zero = torch.zeros_like(step.lens)
            out = kvc.decode_attn_window(step.q, step.k, step.v, zero, step.max_len, window, block_table=step.tbl)
            torch.cuda.synchronize()
            assert torch.count_nonzero(out).item() == 0, "L = 0 must give zeros"


VECTOR_PAGED = {
    # the vector kernel: float32, and bf16 groups of more than 32 heads; its
    # tiles (4 or 8 rows) are shorter than the 16-row split alignment
    "f32_d128": W.WORKLOADS["paged_gqa"].replace(B=4, H_q=16, H_kv=4, d=128, dtype="f32", cached_lo=304,
                                                 cached_hi=304),
    "f32_d256": W.WORKLOADS["paged_gqa"].replace(B=4, H_q=8, H_kv=2, d=256, dtype="f32", cached_lo=304,
                                                 cached_hi=304),
    "bf16_d256_g64": W.WORKLOADS["paged_gqa"].replace(B=4, H_q=64, H_kv=1, d=256, dtype="bf16", cached_lo=304,
                                                      cached_hi=304),
}


@pytest.mark.parametrize("name", sorted(VECTOR_PAGED))
def test_window_vector_kernel_masked_first_tiles(name):
    """Windows whose first token lies 8 to 15 rows past its split's origin (the
    window start rounded down to 16): the first tile of some waves then lies
    wholly before the window, and its rows are all masked."""
    window = 37
    xs = W.draw(VECTOR_PAGED[name])
    w = xs.workload
    xs.cached[:] = torch.tensor([lo + window - 1 for lo in (268, 264, 31, 9)], dtype=torch.int32)
    bs = w.block_size
    for b, c in enumerate(xs.cached.tolist()):        # NaN past each new length
        for t in range(c, xs.block_table.shape[1] * bs):
            blk = int(xs.block_table[b, t // bs])
            if blk >= 0:
                xs.k_cache[blk, :, t % bs] = float("nan")
                xs.v_cache[blk, :, t % bs] = float("nan")
    poison_before_window(xs, window)
    lens = xs.seq_lens.tolist()
    say(f"[window vector kernel {name} W={window}] lens={lens} window starts mod 16="
        f"{[WO.window_start(L, window) % 16 for L in lens]}")
    step = GpuStep(xs)
    k2, v2, q2 = _append_and_check(step, xs)
    ref = oracle_window(xs, k2, v2, q2, window)
    for split in (0, 16, 48, 1 << 20):
        compare_out(_decode_window(step, window, split), ref, w.dtype, f"{name} W={window} split={split}")


def _ring_inputs(B=4, H_q=32, H_kv=8, d=128, T=64, positions=(5, 63, 64, 200), dtype="bf16", seed=31):
    """A ring [B, H_kv, T, d] holding each sequence's window before the step
    (slots of tokens never written are NaN), and the step's raw q / k / v."""
    g = torch.Generator().manual_seed(seed)
    cast = (lambda t: t.to(torch.bfloat16)) if dtype == "bf16" else (lambda t: t)
    ring_k = cast(torch.randn((B, H_kv, T, d), generator=g))
    ring_v = cast(torch.randn((B, H_kv, T, d), generator=g))
    for b, p in enumerate(positions):
        if p < T:                       # slots p .. T-1 never written yet
            ring_k[b, :, p:] = float("nan")
            ring_v[b, :, p:] = float("nan")
    q = cast(torch.randn((B, H_q, d), generator=g))
    kn = cast(torch.randn((B, H_kv, d), generator=g))
    vn = cast(torch.randn((B, H_kv, d), generator=g))
    cos, sin = W.rotation_table(max(positions) + 1, d)
    return ring_k, ring_v, torch.tensor(positions, dtype=torch.int32), q, kn, vn, cos, sin


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_append_and_decode(dtype):
    rk, rv, pos, q, kn, vn, cos, sin = _ring_inputs(dtype=dtype, d=128 if dtype == "bf16" else 64)
    T = rk.shape[2]
    say(f"[ring {dtype}] T={T} positions={pos.tolist()}")
    dev = "cuda"
    k, v, qd = rk.to(dev), rv.to(dev), q.to(dev).clone()
    kvc.append_ring(k, v, pos.to(dev), kn.to(dev), vn.to(dev), cos.to(dev), sin.to(dev), q=qd)
    torch.cuda.synchronize()
    k2, v2, q2 = WO.append_ring(store_np(rk, dtype), store_np(rv, dtype), pos.numpy(), store_np(kn, dtype),
                                store_np(vn, dtype), cos.numpy(), sin.numpy(), dtype, q=store_np(q, dtype))
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "ring K differs from the oracle"
    assert np.array_equal(bits(v), np.ascontiguousarray(v2).view(np.uint8)), "ring V differs from the oracle"
    assert np.array_equal(store_np(qd, dtype).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8))
    lens = pos + 1
    ref = WO.decode_attention_ring(q2, k2, v2, lens.numpy(), dtype)
    for split in (0, 16, 1 << 20):
        out = kvc.decode_attn_window(qd, k, v, lens.to(dev), int(lens.max()), T, ring=True, split_tokens=split)
        torch.cuda.synchronize()
        compare_out(out, ref, dtype, f"ring {dtype} split={split}")


@pytest.mark.parametrize("name", ["gqa_8b", "paged_gqa", "mqa_ragged", "gqa_f32"])
def test_step_window(name):
    """The fused step with a window == oracle append + windowed decode, and ==
    kvc_append + kvc_decode_attn_window bit for bit (gqa_f32: the vector
    kernel, which does the append itself over a contiguous cache)."""
    window = 100
    x = W.draw(SMALL[name])
    poison_before_window(x, window)
    say(f"[step window {name}] lens={x.seq_lens.tolist()[:6]}")
    step = GpuStep(x)
    k, v = step.k.clone(), step.v.clone()
    q_raw = x.q.to("cuda")
    out, q_rot = kvc.decode_step_window(q_raw, k, v, step.pos, step.kn, step.vn, step.cos, step.sin, step.max_len,
                                        window, block_table=step.tbl)
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs from the oracle"
    assert np.array_equal(store_np(q_rot, x.workload.dtype).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8))
    compare_out(out, oracle_window(x, k2, v2, q2, window), x.workload.dtype, f"step {name} W={window}")
    step.append()
    sep = _decode_window(step, window)
    torch.cuda.synchronize()
    assert torch.equal(sep.view(torch.int16), out.view(torch.int16)), "fused step != append + windowed decode"


def test_step_ring():
    rk, rv, pos, q, kn, vn, cos, sin = _ring_inputs()
    T = rk.shape[2]
    dev = "cuda"
    k, v = rk.to(dev), rv.to(dev)
    out, q_rot = kvc.decode_step_window(q.to(dev), k, v, pos.to(dev), kn.to(dev), vn.to(dev), cos.to(dev),
                                        sin.to(dev), int(pos.max()) + 1, T, ring=True)
    torch.cuda.synchronize()
    k2, v2, q2 = WO.append_ring(store_np(rk, "bf16"), store_np(rv, "bf16"), pos.numpy(), store_np(kn, "bf16"),
                                store_np(vn, "bf16"), cos.numpy(), sin.numpy(), "bf16", q=store_np(q, "bf16"))
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "ring K differs from the oracle"
    assert np.array_equal(store_np(q_rot, "bf16").view(np.uint8), np.ascontiguousarray(q2).view(np.uint8))
    compare_out(out, WO.decode_attention_ring(q2, k2, v2, (pos + 1).numpy(), "bf16"), "bf16", "ring step")


def test_window_full_size():
    """gqa_8b at full size (16 x 8193 tokens) with a 4096-token window, through
    the fused step in the library's launch plan, every output compared."""
    w = W.WORKLOADS["gqa_8b"]
    window = 4096
    x = W.draw(w)
    poison_before_window(x, window)
    say(f"[window full gqa_8b W={window}]")
    step = GpuStep(x)
    k, v = step.k, step.v
    out, q_rot = kvc.decode_step_window(x.q.to("cuda"), k, v, step.pos, step.kn, step.vn, step.cos, step.sin,
                                        step.max_len, window)
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(q_rot), np.ascontiguousarray(q2).view(np.uint8)), "rotated q differs"
    compare_out(out, oracle_window(x, k2, v2, q2, window), w.dtype, f"gqa_8b W={window} full size")