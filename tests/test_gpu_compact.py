"""The compacted schedule of the bf16 matrix-core kernel (contiguous caches
whose split plan would take several rounds) on the GPU, against the oracle.

Under that schedule every workgroup reads all B lengths, picks the split
length from them (the shortest multiple of the loop step whose splits of all
units fit in one round) and takes the split that its index names in unit
order; the merge kernel derives the same length and combines the splits.
These cases cover what can go wrong there: ragged and degenerate lengths
(1, 2, one step, a step plus one, the longest), groups of 24 and 32 heads
(two 16-head blocks), one and two KV heads, head_dim 64, 128 and 256, a
sliding window, uniform lengths, the fused step (the rotated
query written by split 0, the new token stored by the unit's last split),
bitwise determinism over a workspace full of garbage (partial slots past a
sequence's splits are never read), and the arrival counters left at zero.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import oracle.kvc_window_oracle as WO
import workloads as W
from gpu_helpers import GpuStep, bits, compare_out, oracle_append, oracle_decode, run_step, say, store_np

pytestmark = pytest.mark.gpu


def _draw(B, H_q, H_kv, d, lens, seed):
    """A contiguous bf16 workload with these attended lengths (cached = L - 1),
    NaN at and past each sequence's cached length."""
    T_max = (max(lens) + 15) // 8 * 8
    w = W.WORKLOADS["mqa_ragged"].replace(seed=seed, B=B, H_q=H_q, H_kv=H_kv, d=d, cached_lo=max(lens) - 1,
                                          cached_hi=max(lens) - 1, T_max=T_max)
    x = W.draw(w)
    x.cached[:] = torch.tensor([L - 1 for L in lens], dtype=torch.int32)
    for b, c in enumerate(x.cached.tolist()):
        x.k_cache[b, :, c:] = float("nan")
        x.v_cache[b, :, c:] = float("nan")
    return x


def _garbage_workspace(w, max_len, window=0):
    span = kvc.window_span(max_len, window) if window else max_len
    n = kvc.workspace_bytes(torch.bfloat16, w.B, w.H_q, w.H_kv, w.d, span)
    ws = torch.full((max(n, 256),), 0x7F, dtype=torch.uint8, device="cuda")
    ws[:kvc.workspace_zeroed_bytes()].zero_()
    return ws


def _check(B, H_q, H_kv, d, lens, seed, label):
    x = _draw(B, H_q, H_kv, d, lens, seed)
    w = x.workload
    step = GpuStep(x)
    assert kvc.compact(torch.bfloat16, B, H_q, H_kv, d, step.max_len), "expected the compacted schedule"
    assert kvc.merge_launch(torch.bfloat16, B, H_q, H_kv, d, step.max_len)
    say(f"[compact {label}] B={B} H_q={H_q} H_kv={H_kv} d={d} lens={x.seq_lens.tolist()[:10]}")
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    assert np.array_equal(bits(step.k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs"
    assert np.array_equal(bits(step.v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs"
    ref = oracle_decode(x, k2, v2, q2)
    ws = _garbage_workspace(w, step.max_len)
    out = kvc.decode_attn(step.q, step.k, step.v, step.lens, step.max_len, workspace=ws)
    again = kvc.decode_attn(step.q, step.k, step.v, step.lens, step.max_len, workspace=ws)
    torch.cuda.synchronize()
    compare_out(out, ref, "bf16", f"{label} decode")
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "run-to-run difference"
    assert int(torch.count_nonzero(ws[:kvc.workspace_zeroed_bytes()])) == 0, "arrival counters left nonzero"
    # the fused step on fresh copies of the inputs: cache, rotated query and output
    k, v, q_rot, out_s = run_step(step)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "step: K cache differs"
    assert np.array_equal(bits(v), np.ascontiguousarray(v2).view(np.uint8)), "step: V cache differs"
    assert np.array_equal(store_np(q_rot, "bf16").view(np.uint8), np.ascontiguousarray(q2).view(np.uint8)), \
        "step: rotated q differs"
    compare_out(out_s, ref, "bf16", f"{label} step")
    return x, step, (k2, v2, q2)


def test_mqa_32_heads_edge_lengths():
    _check(8, 32, 1, 128, [1, 2, 64, 65, 4097, 9000, 12000, 16001], 101, "mqa d128")


def test_two_kv_heads_d64():
    rnd = np.random.default_rng(7)
    lens = [20001] + rnd.integers(1, 20001, 5).tolist()
    _check(6, 64, 2, 64, lens, 102, "G32 H_kv2 d64")


def test_24_heads_d256():
    rnd = np.random.default_rng(8)
    lens = [14001, 1, 129, 128] + rnd.integers(1, 14001, 4).tolist()
    _check(8, 24, 1, 256, lens, 103, "G24 d256")


def test_many_short_sequences():
    rnd = np.random.default_rng(9)
    lens = [6001] + rnd.integers(1, 6001, 39).tolist()
    _check(40, 32, 1, 128, lens, 104, "40 seqs")


def test_uniform_lengths():
    _check(8, 32, 1, 128, [16385] * 8, 105, "uniform")


def test_window():
    lens = [1, 65, 3000, 9000, 12000, 15000, 16001, 14001]
    x = _draw(8, 32, 1, 128, lens, 106)
    window = 14000
    for b, L in enumerate(x.seq_lens.tolist()):
        lo = WO.window_start(L, window)
        x.k_cache[b, :, :lo] = float("nan")
        x.v_cache[b, :, :lo] = float("nan")
    step = GpuStep(x)
    span = kvc.window_span(step.max_len, window)
    assert kvc.compact(torch.bfloat16, 8, 32, 1, 128, span), "expected the compacted schedule"
    say(f"[compact window {window}] lens={lens}")
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    ref = WO.decode_attention_window(q2, k2, v2, x.seq_lens.numpy(), window, "bf16")
    out = kvc.decode_attn_window(step.q, step.k, step.v, step.lens, step.max_len, window)
    torch.cuda.synchronize()
    compare_out(out, ref, "bf16", f"window {window}")
