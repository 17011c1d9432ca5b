"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Append: bit-exact over the whole cache buffers and the rotated query.
Attention: max-abs error <= 2e-3 (bf16; the oracle rounded to bf16) and
<= 1e-5 (float32), at oracle-sized shapes that span many tiles and splits with
ragged tails, and at the workloads' full sizes on every output, in the launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import GpuStep, bits, compare_out, oracle_append, oracle_decode, say, store_np

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_mha": W.WORKLOADS["tiny_mha"],
    "gqa_8b": W.WORKLOADS["gqa_8b"].replace(B=3, cached_lo=300, cached_hi=1100, T_max=1104),
    "mqa_ragged": W.WORKLOADS["mqa_ragged"].replace(B=5, cached_lo=100, cached_hi=700, T_max=704),
    "long_gqa": W.WORKLOADS["long_gqa"].replace(cached_lo=3000, cached_hi=3000, T_max=3008),
    "paged_gqa": W.WORKLOADS["paged_gqa"].replace(B=4, cached_lo=20, cached_hi=400),
}


def _check_append(step: GpuStep, x, style="interleaved"):
    k2, v2, q2 = oracle_append(x, style)
    dt = x.workload.dtype
    assert np.array_equal(bits(step.k), np.ascontiguousarray(k2).view(np.uint8)), "K cache differs from the oracle"
    assert np.array_equal(bits(step.v), np.ascontiguousarray(v2).view(np.uint8)), "V cache differs from the oracle"
    assert np.array_equal(store_np(step.q, dt).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8)), \
        "rotated q differs from the oracle"
    return k2, v2, q2


@pytest.mark.parametrize("name", sorted(SMALL))
def test_step_matches_oracle(name):
    x = W.draw(SMALL[name])
    say(f"[{name}] B={x.workload.B} lens={x.seq_lens.tolist()[:6]} append+decode")
    step = GpuStep(x)
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = _check_append(step, x)
    ref = oracle_decode(x, k2, v2, q2)
    for split in (0, 64, 100, 1 << 20):
        out = step.decode(split_tokens=split)
        torch.cuda.synchronize()
        compare_out(out, ref, x.workload.dtype, f"{name} split_tokens={split}")


@pytest.mark.parametrize("name", ["gqa_8b", "paged_gqa", "tiny_mha"])
def test_half_rotation_style(name):
    x = W.draw(SMALL[name])
    say(f"[{name}] rope_style=half")
    step = GpuStep(x)
    step.append(rope_style="half")
    torch.cuda.synchronize()
    k2, v2, q2 = _check_append(step, x, "half")
    compare_out(step.decode(), oracle_decode(x, k2, v2, q2), x.workload.dtype, f"{name} half")


def test_edge_lengths():
    """L = 1 (empty cache before the step), L = 0, tile-exact and tile+1 lengths."""
    base = W.WORKLOADS["gqa_8b"].replace(B=6, cached_lo=511, cached_hi=511, T_max=520)
    x = W.draw(base)
    x.cached[:] = torch.tensor([0, 63, 64, 127, 255, 511], dtype=torch.int32)
    # re-poison so slots >= cached are NaN for the new lengths
    for b, c in enumerate(x.cached.tolist()):
        x.k_cache[b, :, c:] = float("nan")
        x.v_cache[b, :, c:] = float("nan")
    say(f"[edge] lens={x.seq_lens.tolist()}")
    step = GpuStep(x)
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = _check_append(step, x)
    ref = oracle_decode(x, k2, v2, q2)
    for split in (0, 64, 1 << 20):
        compare_out(step.decode(split_tokens=split), ref, "bf16", f"edge split={split}")
    # one token: the output is exactly that token's value (a single weight of 1)
    out = step.decode()
    torch.cuda.synchronize()
    vn = store_np(x.v_new, "bf16")
    assert np.array_equal(store_np(out, "bf16")[0].reshape(8, 4, 128)[:, 0], vn[0])
    # L = 0 for every sequence: zeros
    zero = torch.zeros_like(step.lens)
    out0 = step.decode(lens=zero, max_len=0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out0.float()) == 0


def test_split_invariance_and_determinism():
    x = W.draw(SMALL["long_gqa"])
    say("[long_gqa small] split invariance")
    step = GpuStep(x)
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = _check_append(step, x)
    ref = oracle_decode(x, k2, v2, q2)
    outs = {}
    for split in (16, 64, 200, 1500, 3001, 0):
        outs[split] = step.decode(split_tokens=split).clone()
        torch.cuda.synchronize()
        compare_out(outs[split], ref, "bf16", f"split={split}")
    again = step.decode(split_tokens=64)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), outs[64].view(torch.int16)), "run-to-run difference"


def test_nondefault_stream():
    x = W.draw(SMALL["gqa_8b"])
    say("[gqa_8b small] side stream")
    step = GpuStep(x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step.append(stream=s)
        out = step.decode(stream=s)
    s.synchronize()
    k2, v2, q2 = _check_append(step, x)
    compare_out(out, oracle_decode(x, k2, v2, q2), "bf16", "side stream")


def test_stream_argument_outside_its_context():
    """stream= given without making that stream current: the calls run there,
    and the workspace the binding grows for the second (longer) call belongs
    to that stream, so both results are right."""
    s = torch.cuda.Stream()
    for i, (w, split) in enumerate(((SMALL["gqa_8b"], 64), (SMALL["long_gqa"], 16))):
        x = W.draw(w)
        say(f"[side stream, not current] {w.name} split={split}")
        step = GpuStep(x)
        s.wait_stream(torch.cuda.current_stream())
        step.append(stream=s)
        out = step.decode(split_tokens=split, stream=s)
        s.synchronize()
        k2, v2, q2 = _check_append(step, x)
        compare_out(out, oracle_decode(x, k2, v2, q2), w.dtype, f"side stream call {i}")


def test_paged_equals_contiguous():
    """The same logical cache as a contiguous buffer and as a shuffled block pool.

    The two kernels add the tokens in different orders (the contiguous one
    spreads each 16-token group over its four waves, the paged one gives each
    wave 32 consecutive tokens), so they agree to float32 rounding: after the
    bf16 store most outputs are equal, and the rest differ where the float32
    result lies near a bf16 rounding midpoint - one step, two across a power
    of two - or where the output is a cancellation far below its terms (there
    float32 rounding of terms of size ~0.1 is a few 1e-8, several bf16 steps of
    a 1e-5 output).  A wrong block or row gives errors far larger and far more
    frequent.  Both are also checked against the oracle elsewhere."""
    w = W.WORKLOADS["gqa_8b"].replace(B=4, cached_lo=50, cached_hi=900, T_max=912)
    x = W.draw(w)
    say("[paged == contiguous]")
    step = GpuStep(x)
    step.append()
    torch.cuda.synchronize()
    bs = 16
    B, H_kv, T, d = step.k.shape
    nblk = -(-T // bs)
    g = torch.Generator().manual_seed(11)
    perm = torch.randperm(B * nblk, generator=g)
    table = perm.view(B, nblk).to(torch.int32)
    kp = torch.empty((B * nblk, H_kv, bs, d), dtype=step.k.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kpad = torch.nn.functional.pad(step.k, (0, 0, 0, nblk * bs - T))
    vpad = torch.nn.functional.pad(step.v, (0, 0, 0, nblk * bs - T))
    kp[table.flatten().long().cuda()] = kpad.view(B, H_kv, nblk, bs, d).permute(0, 2, 1, 3, 4).reshape(-1, H_kv, bs, d)
    vp[table.flatten().long().cuda()] = vpad.view(B, H_kv, nblk, bs, d).permute(0, 2, 1, 3, 4).reshape(-1, H_kv, bs, d)
    import mqa_decode_attention_amd as kvc
    for split in (0, 128):
        a = kvc.decode_attn(step.q, step.k, step.v, step.lens, step.max_len, split_tokens=split)
        p = kvc.decode_attn_paged(step.q, kp, vp, table.cuda(), step.lens, step.max_len, split_tokens=split)
        torch.cuda.synchronize()
        af, pf = a.float(), p.float()
        big = torch.maximum(af.abs(), pf.abs()).clamp(min=2.0 ** -126)
        step_ = big.frexp().exponent.float().sub(8).exp2()        # one bf16 step at the larger magnitude
        diff = (af - pf).abs()
        same = float((diff == 0).float().mean())
        say(f"  split {split}: equal {same:.4f}, max diff {float(diff.max()):.3g}, mean diff {float(diff.mean()):.3g}")
        bad = diff > 2 * step_ + 2e-6
        assert not bool(bad.any()), f"paged vs contiguous (split {split}): {int(bad.sum())} outputs differ beyond rounding"
        assert float(diff.mean()) < 1e-5, f"paged vs contiguous (split {split}): mean diff {float(diff.mean())}"
        assert same > 0.95, f"paged vs contiguous (split {split}): only {same:.3f} of outputs equal"


# ---------------------------------------------------------------------------
# full sizes, default launch plan (what the benchmark times)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["gqa_8b", "mqa_ragged", "long_gqa", "paged_gqa"])
def test_full_size(name):
    """Every output at the workload's full size, in the default launch plan."""
    w = W.WORKLOADS[name]
    x = W.draw(w)
    say(f"[{name} full] B={w.B} max_len={int(x.seq_lens.max())}")
    step = GpuStep(x)
    step.append()
    out = step.decode()
    torch.cuda.synchronize()
    # the append, over the whole buffers
    k2, v2, q2 = _check_append(step, x)
    # attention: every (sequence, query head) row
    compare_out(out, oracle_decode(x, k2, v2, q2), w.dtype, f"{name} full size")


def test_workspace_reuse_across_shapes():
    """One workspace buffer shared by calls of different shapes, filled with
    garbage first past its zeroed prefix (the arrival counters): no call may
    depend on what an earlier call left in it, and every call leaves the
    counters at zero."""
    import mqa_decode_attention_amd as kvc
    ws = torch.full((64 << 20,), 0x7F, dtype=torch.uint8, device="cuda")
    zb = kvc.workspace_zeroed_bytes()
    assert zb > 0 and zb % 256 == 0
    ws[:zb].zero_()
    cases = [SMALL["long_gqa"], SMALL["mqa_ragged"], SMALL["gqa_8b"], SMALL["long_gqa"]]
    for i, w in enumerate(cases):
        x = W.draw(w)
        say(f"[workspace reuse {i}] {w.name}")
        step = GpuStep(x)
        step.append()
        for split in (16, 64):
            out = kvc.decode_attn(step.q, step.k, step.v, step.lens, step.max_len, split_tokens=split,
                                  workspace=ws)
            torch.cuda.synchronize()
            k2, v2, q2 = oracle_append(x)
            compare_out(out, oracle_decode(x, k2, v2, q2), w.dtype, f"reuse {w.name} split={split}")
            assert int(torch.count_nonzero(ws[:zb])) == 0, "arrival counters left nonzero"


GROUP_CASES = [
    # (H_q, H_kv, d, dtype): MHA, odd and large groups, every head_dim, both dtypes
    (8, 8, 128, "bf16"), (12, 4, 128, "bf16"), (16, 1, 128, "bf16"), (24, 1, 128, "bf16"),
    (48, 2, 128, "bf16"), (8, 2, 64, "bf16"), (8, 2, 256, "bf16"), (64, 2, 256, "bf16"),
    (8, 2, 32, "bf16"), (4, 4, 16, "bf16"), (16, 4, 128, "f32"), (6, 2, 16, "f32"), (64, 2, 64, "f32"),
    # groups beyond 32 heads in bf16 (vector kernel, several head chunks)
    (64, 1, 128, "bf16"), (96, 2, 64, "bf16"),
]


@pytest.mark.parametrize("H_q,H_kv,d,dtype", GROUP_CASES)
def test_group_shapes(H_q, H_kv, d, dtype):
    w = W.Workload("groups", 21, B=3, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, cached_lo=90, cached_hi=700,
                   T_max=704)
    x = W.draw(w)
    say(f"[groups] H_q={H_q} H_kv={H_kv} d={d} {dtype} lens={x.seq_lens.tolist()}")
    step = GpuStep(x)
    step.append()
    torch.cuda.synchronize()
    k2, v2, q2 = _check_append(step, x)
    ref = oracle_decode(x, k2, v2, q2)
    for split in (0, 96, 1 << 20):
        compare_out(step.decode(split_tokens=split), ref, dtype, f"G={H_q // H_kv} d={d} {dtype} split={split}")
