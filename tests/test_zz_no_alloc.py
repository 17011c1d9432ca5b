"""kvc_decode_step_noalloc on the GPU, through the C ABI: the same append and
attention as kvc_decode_step (its partials in the library's fixed device array
instead of a caller's workspace).

Two calls in a row, the second with a smaller input (fewer sequences, shorter
caches, another split plan), each against kvc_decode_step on identical copies
of the inputs: caches and rotated queries bit for bit, outputs within the
attention bar of the oracle parity tests (2e-3 max abs for bf16, 1e-5 for
float32) - and also equal to them bit for bit, since both run the same kernels
on the same plan.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import workloads as W
from gpu_helpers import BF16_TOL, F32_TOL, GpuStep, bits, run_step, say

pytestmark = pytest.mark.gpu

CALLS = [
    # (workload, split_tokens): a larger call, then a smaller one
    (W.WORKLOADS["gqa_8b"].replace(B=4, cached_lo=900, cached_hi=2100, T_max=2104), 0),
    (W.WORKLOADS["gqa_8b"].replace(B=2, cached_lo=100, cached_hi=600, T_max=608), 128),
    (W.WORKLOADS["paged_gqa"].replace(B=3, cached_lo=200, cached_hi=900), 0),
    (W.WORKLOADS["tiny_mha"], 0),
]


def _noalloc(step: GpuStep, split: int):
    x = step.x
    k, v = step.k.clone(), step.v.clone()
    q = x.q.to(step.k.device)
    out, q_rot = torch.empty_like(q), torch.empty_like(q)
    kvc.decode_step_noalloc(q, k, v, step.pos, step.kn, step.vn, step.cos, step.sin, step.max_len, q_rot, out,
                            block_table=step.tbl, split_tokens=split)
    return k, v, q_rot, out


def test_noalloc_step_matches_decode_step():
    for i, (w, split) in enumerate(CALLS):
        x = W.draw(w)
        say(f"[noalloc call {i}] {w.name} B={w.B} max_len={int(x.seq_lens.max())} split={split}")
        step = GpuStep(x)
        k1, v1, q1, o1 = run_step(step, split_tokens=split)
        k2, v2, q2, o2 = _noalloc(step, split)
        torch.cuda.synchronize()
        assert np.array_equal(bits(k1), bits(k2)), "K cache differs"
        assert np.array_equal(bits(v1), bits(v2)), "V cache differs"
        assert np.array_equal(bits(q1), bits(q2)), "rotated query differs"
        err = float((o1.double() - o2.double()).abs().max())
        tol = BF16_TOL if w.dtype == "bf16" else F32_TOL
        say(f"  max|out - kvc_decode_step out| = {err:.3g} (tol {tol})")
        assert err <= tol
        assert np.array_equal(bits(o1), bits(o2)), "output differs from kvc_decode_step"


def test_noalloc_rejects_sizes_beyond_its_array():
    w = W.WORKLOADS["gqa_8b"].replace(B=2, cached_lo=100, cached_hi=100, T_max=128)
    x = W.draw(w)
    step = GpuStep(x)
    q = x.q.to("cuda")
    out, q_rot = torch.empty_like(q), torch.empty_like(q)
    need = kvc.workspace_bytes(q.dtype, 64, 64, 8, 128, 4096, 16)
    assert need > kvc.noalloc_max_bytes()
    B, H_q, d = 64, 64, 128
    big_q = torch.zeros((B, H_q, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, 8, 4096, d), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, 8, d), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_step_noalloc(big_q, kc, kc, pos, kn, kn, step.cos, step.sin, 4096, torch.empty_like(big_q),
                                torch.empty_like(big_q), split_tokens=16)
    assert e.value.status == 4 and "scratch" in str(e.value)
    torch.cuda.synchronize()
