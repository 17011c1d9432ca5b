"""The balanced schedule of the bf16 matrix-core kernel (ragged paged pools)
on the GPU, against the oracle.

Under that schedule every workgroup streams an equal share of all units'
loop steps, so a unit's tokens may be split among several workgroups at
arbitrary 64-token boundaries and merged by the last of them to finish.
These cases cover what can go wrong there: ragged and degenerate lengths
(0, 1, one step, a step plus one, block boundaries), fewer steps than
workgroups, one long sequence spread over hundreds of workgroups, groups of
4, 24 and 32 heads (one and two 16-head blocks), head_dim 64 and 128, block
sizes 16 and 32, the fused step (the new token owned by the unit's last
workgroup, the rotated query written by its first), bitwise determinism and
the arrival counters left at zero.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import workloads as W
from gpu_helpers import GpuStep, bits, compare_out, oracle_append, oracle_decode, run_step, say

pytestmark = pytest.mark.gpu


def _pool_tokens(step):
    return 0 if step.tbl is None else int(step.k.shape[0]) * step.x.workload.block_size


def _assert_balanced(step, max_len=None):
    w = step.x.workload
    ml = step.max_len if max_len is None else max_len
    assert kvc.balanced(torch.bfloat16, w.B, w.H_q, w.H_kv, w.d, ml, pool_tokens=_pool_tokens(step)), \
        "expected the balanced schedule for these sizes"


def _check(w, lens_override=None, label=""):
    x = W.draw(w)
    step = GpuStep(x)
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x)
    _assert_balanced(step)
    say(f"[balanced {label}] B={w.B} G={w.H_q // w.H_kv} d={w.d} lens={x.seq_lens.tolist()[:12]}")
    zb = kvc.workspace_zeroed_bytes()
    ws = torch.full((kvc.workspace_bytes(torch.bfloat16, w.B, w.H_q, w.H_kv, w.d, step.max_len,
                                         pool_tokens=_pool_tokens(step)),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    ws[:zb].zero_()
    if step.tbl is not None:
        out = kvc.decode_attn_paged(step.q, step.k, step.v, step.tbl, step.lens, step.max_len, workspace=ws)
    else:
        out = kvc.decode_attn(step.q, step.k, step.v, step.lens, step.max_len, workspace=ws)
    again = step.decode()
    torch.cuda.synchronize()
    compare_out(out, oracle_decode(x, k2, v2, q2), "bf16", f"{label} library plan")
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "run-to-run difference"
    assert int(torch.count_nonzero(ws[:zb])) == 0, "arrival counters left nonzero"
    if lens_override is not None:
        lens = np.minimum(np.asarray(lens_override, np.int32), x.seq_lens.numpy())
        say(f"  shortened lens={lens.tolist()[:12]}")
        t = torch.from_numpy(lens).cuda()
        o2 = step.decode(lens=t)
        torch.cuda.synchronize()
        compare_out(o2, oracle_decode(x, k2, v2, q2, seq_lens=lens), "bf16", f"{label} shortened")


def test_group32_ragged():
    w = W.Workload("bal_g32", 41, B=9, H_q=32, H_kv=1, d=128, dtype="bf16", cached_lo=1, cached_hi=1400,
                   layout="paged", block_size=16)
    _check(w, [0, 1, 63, 64, 65, 128, 700, 5, 2], "G=32 d=128")


def test_group24_d64():
    w = W.Workload("bal_g24", 42, B=7, H_q=48, H_kv=2, d=64, dtype="bf16", cached_lo=0, cached_hi=900,
                   layout="paged", block_size=16)
    _check(w, [0, 64, 1, 129, 900, 300, 64], "G=24 d=64")


def test_fewer_steps_than_workgroups():
    """Three sequences shortened to 1, 0 and 2 tokens: 3 steps for 512
    planned workgroups."""
    w = W.Workload("bal_tiny", 43, B=3, H_q=8, H_kv=1, d=128, dtype="bf16", cached_lo=0, cached_hi=300,
                   layout="paged", block_size=16)
    _check(w, [1, 0, 2], "fewer steps")


def test_one_long_sequence_over_many_workgroups():
    """One long sequence beside a 1-token one under one KV head of 32 query
    heads: its ~300 steps fall to ~300 workgroups, each contributing a
    partial to one merge."""
    w = W.Workload("bal_long", 44, B=2, H_q=32, H_kv=1, d=128, dtype="bf16", cached_lo=0, cached_hi=20000,
                   layout="paged", block_size=16)
    _check(w, [1, 20001], "one long")


def test_ragged_pool_gqa():
    w = W.Workload("bal_paged", 45, B=12, H_q=32, H_kv=8, d=128, dtype="bf16", cached_lo=1, cached_hi=3000,
                   layout="paged", block_size=16)
    _check(w, [0, 1, 16, 17, 63, 64, 65, 2000, 3, 1000, 128, 129], "G=4 d=128")


def test_ragged_pool_d64_block32():
    w = W.Workload("bal_paged64", 46, B=10, H_q=16, H_kv=4, d=64, dtype="bf16", cached_lo=0, cached_hi=2500,
                   layout="paged", block_size=32)
    _check(w, [5, 0, 64, 31, 32, 33, 2500, 100, 1, 700], "G=4 d=64 bs=32")


STEP_CASES = {
    "g32": W.Workload("bal_step_g32", 47, B=6, H_q=32, H_kv=1, d=128, dtype="bf16", cached_lo=0, cached_hi=1300,
                      layout="paged", block_size=16),
    "g4": W.Workload("bal_step_g4", 48, B=9, H_q=32, H_kv=8, d=128, dtype="bf16", cached_lo=0, cached_hi=2000,
                     layout="paged", block_size=16),
}


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("name", sorted(STEP_CASES))
def test_fused_step(name, style):
    """kvc_decode_step under the balanced schedule: bit-exact append and
    rotated query, attention within tolerance, and bitwise equal to
    kvc_append followed by kvc_decode_attn (the same schedule)."""
    x = W.draw(STEP_CASES[name])
    say(f"[balanced step {name} {style}] lens={x.seq_lens.tolist()}")
    s = GpuStep(x)
    _assert_balanced(s)
    k, v, q_rot, out = run_step(s, rope_style=style)
    a = GpuStep(x)
    a.append(rope_style=style)
    out_a = a.decode()
    torch.cuda.synchronize()
    k2, v2, q2 = oracle_append(x, style)
    assert np.array_equal(bits(k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs from the oracle"
    assert np.array_equal(bits(q_rot), np.ascontiguousarray(q2).view(np.uint8)), "rotated q differs"
    compare_out(out, oracle_decode(x, k2, v2, q2), "bf16", f"step {name} {style}")
    assert np.array_equal(bits(out), bits(out_a)), "step output differs from append + decode"


# ---- the quantized (uint8) cache under the same schedule (128-token steps)

U8_CASES = {
    "g4": W.Workload("bal_u8_g4", 51, B=12, H_q=32, H_kv=8, d=128, dtype="bf16", cached_lo=1, cached_hi=3000,
                     layout="paged", block_size=16),
    "g32_d64": W.Workload("bal_u8_g32", 52, B=7, H_q=32, H_kv=1, d=64, dtype="bf16", cached_lo=0, cached_hi=2500,
                          layout="paged", block_size=32),
}


@pytest.mark.parametrize("name", sorted(U8_CASES))
def test_u8_ragged_pool(name):
    from test_gpu_quant import QStep, check_append
    import oracle.kvc_quant_oracle as QO
    w = U8_CASES[name]
    x = W.draw(w)
    qc = W.draw_quantized(x)
    s = QStep(x, qc)
    pool = int(s.kc.shape[0]) * w.block_size
    assert kvc.balanced(torch.uint8, w.B, w.H_q, w.H_kv, w.d, s.max_len, pool_tokens=pool), \
        "expected the balanced schedule for these sizes"
    say(f"[balanced u8 {name}] B={w.B} G={w.H_q // w.H_kv} d={w.d} lens={x.seq_lens.tolist()[:12]}")
    s.append()
    torch.cuda.synchronize()
    kc, ks, vc, vs, q2 = check_append(s, x, qc)
    tbl = x.block_table.numpy()
    full = x.seq_lens.numpy()
    short = np.minimum(np.array([0, 1, 127, 128, 129, 2000, 16, 17, 3, 1000, 256, 257][:w.B], np.int32), full)
    for lens in (full, short):
        t = torch.from_numpy(np.ascontiguousarray(lens)).cuda()
        out = kvc.decode_attn_paged_u8(s.q, s.kc, s.ks, s.vc, s.vs, s.tbl, t, s.max_len)
        again = kvc.decode_attn_paged_u8(s.q, s.kc, s.ks, s.vc, s.vs, s.tbl, t, s.max_len)
        torch.cuda.synchronize()
        ref = QO.decode_attention_paged_u8(q2, kc, ks, vc, vs, tbl, w.block_size, lens, "bf16")
        compare_out(out, ref, "bf16", f"u8 {name} lens={lens.tolist()[:6]}")
        assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "run-to-run difference"


@pytest.mark.parametrize("name", sorted(U8_CASES))
def test_u8_fused_step(name):
    """kvc_decode_step_u8 under the balanced schedule: bitwise equal to
    kvc_append_u8 then kvc_decode_attn_paged_u8 (same schedule), the append
    bit-exact against the oracle, attention within tolerance."""
    from test_gpu_quant import QStep, check_append, _run_step_u8
    import oracle.kvc_quant_oracle as QO
    w = U8_CASES[name]
    x = W.draw(w)
    qc = W.draw_quantized(x)
    say(f"[balanced u8 step {name}] lens={x.seq_lens.tolist()[:12]}")
    ref = QStep(x, qc)
    ref.append()
    torch.cuda.synchronize()
    kc2, ks2, vc2, vs2, q2 = check_append(ref, x, qc)
    kc, ks, vc, vs, q_rot, out = _run_step_u8(QStep(x, qc))
    out_a = ref.decode()
    torch.cuda.synchronize()
    for what, got, exp in (("K codes", kc, ref.kc), ("K pairs", ks, ref.ks), ("V codes", vc, ref.vc),
                           ("V pairs", vs, ref.vs), ("rotated q", q_rot, ref.q)):
        assert np.array_equal(bits(got), bits(exp)), f"{what} differ from the append"
    assert np.array_equal(bits(out), bits(out_a)), "output differs from append + decode"
    oref = QO.decode_attention_paged_u8(q2, kc2, ks2, vc2, vs2, x.block_table.numpy(), w.block_size,
                                        x.seq_lens.numpy(), "bf16")
    compare_out(out, oref, "bf16", f"u8 step {name}")
