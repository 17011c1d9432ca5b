"""GPU parity of the quantized-cache path (uint8 codes with a (step, zero point)
pair per cached vector) with its oracle, through the C ABI.

* kvc_append_u8 must give the oracle's codes, pairs and rotated query bit for
  bit (the codes are integers decided in float32 by both sides).
* kvc_decode_attn[_paged]_u8 must match the oracle's float64 attention over
  the dequantized values within 2e-3 after bf16 rounding, for several splits
  (including ones that leave waves without a tile), both layouts, head_dim 64
  and 128, groups of 4 to 32 heads, and at the workloads' full sizes on
  sampled (sequence, KV head) groups in the launch configuration of the
  library's plan.

Inputs: the workloads' seeded draws for the queries and new tokens, and
quantized caches drawn by workloads.draw_quantized.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import oracle as O
import oracle.kvc_quant_oracle as QO
import workloads as W
from gpu_helpers import BF16_TOL, bits, compare_out, say, store_np

pytestmark = pytest.mark.gpu

SMALL = {
    "gqa_8b": W.WORKLOADS["gqa_8b"].replace(B=3, cached_lo=300, cached_hi=1100, T_max=1104),
    "mqa_ragged": W.WORKLOADS["mqa_ragged"].replace(B=5, cached_lo=100, cached_hi=700, T_max=704),
    "long_gqa": W.WORKLOADS["long_gqa"].replace(cached_lo=3000, cached_hi=3000, T_max=3008),
    "paged_gqa": W.WORKLOADS["paged_gqa"].replace(B=4, cached_lo=20, cached_hi=400),
    "gqa_d64": W.WORKLOADS["gqa_8b"].replace(B=2, d=64, cached_lo=150, cached_hi=500, T_max=504),
    "paged_mqa": W.WORKLOADS["paged_gqa"].replace(B=3, H_q=24, H_kv=1, cached_lo=50, cached_hi=300),
}


class QStep:
    def __init__(self, x: W.DecodeInputs, qc: W.QuantCache, device="cuda"):
        w = x.workload
        self.x = x
        self.kc, self.ks = qc.k_codes.to(device), qc.k_sz.to(device)
        self.vc, self.vs = qc.v_codes.to(device), qc.v_sz.to(device)
        self.q = x.q.to(device).clone()
        self.kn, self.vn = x.k_new.to(device), x.v_new.to(device)
        self.pos = x.cached.to(device)
        self.lens = x.seq_lens.to(device)
        self.cos, self.sin = x.rope_cos.to(device), x.rope_sin.to(device)
        self.tbl = x.block_table.to(device) if w.paged else None
        self.max_len = int(x.seq_lens.max())

    def append(self, style="interleaved"):
        kvc.append_u8(self.kc, self.ks, self.vc, self.vs, self.pos, self.kn, self.vn, self.cos, self.sin,
                      q=self.q, block_table=self.tbl, rope_style=style)

    def decode(self, split_tokens=0):
        if self.tbl is not None:
            return kvc.decode_attn_paged_u8(self.q, self.kc, self.ks, self.vc, self.vs, self.tbl, self.lens,
                                            self.max_len, split_tokens=split_tokens)
        return kvc.decode_attn_u8(self.q, self.kc, self.ks, self.vc, self.vs, self.lens, self.max_len,
                                  split_tokens=split_tokens)


def oracle_append_u8(x, qc, style="interleaved"):
    w = x.workload
    dt = w.dtype
    arrs = (qc.k_codes.numpy(), qc.k_sz.numpy(), qc.v_codes.numpy(), qc.v_sz.numpy())
    q, kn, vn = store_np(x.q, dt), store_np(x.k_new, dt), store_np(x.v_new, dt)
    cos, sin = x.rope_cos.numpy(), x.rope_sin.numpy()
    cached = x.cached.numpy()
    if w.paged:
        return QO.append_paged_u8(*arrs, x.block_table.numpy(), w.block_size, cached, kn, vn, cos, sin, dt,
                                  style, q=q)
    return QO.append_contiguous_u8(*arrs, cached, kn, vn, cos, sin, dt, style, q=q)


def check_append(step: QStep, x, qc, style="interleaved"):
    kc, ks, vc, vs, q2 = oracle_append_u8(x, qc, style)
    for name, got, ref in (("K codes", step.kc, kc), ("K pairs", step.ks, ks), ("V codes", step.vc, vc),
                           ("V pairs", step.vs, vs)):
        assert np.array_equal(bits(got), np.ascontiguousarray(ref).view(np.uint8)), f"{name} differ from the oracle"
    assert np.array_equal(store_np(step.q, x.workload.dtype).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8)), \
        "rotated q differs from the oracle"
    return kc, ks, vc, vs, q2


def compare(got: torch.Tensor, ref64: np.ndarray, what: str):
    compare_out(got, ref64, "bf16", what)


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_append_u8_bit_exact(name, style):
    x = W.draw(SMALL[name])
    qc = W.draw_quantized(x)
    say(f"[append_u8 {name} {style}] lens={x.seq_lens.tolist()[:6]}")
    step = QStep(x, qc)
    step.append(style)
    torch.cuda.synchronize()
    check_append(step, x, qc, style)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_u8_matches_oracle(name):
    x = W.draw(SMALL[name])
    w = x.workload
    qc = W.draw_quantized(x)
    say(f"[decode_u8 {name}] G={w.G} d={w.d} lens={x.seq_lens.tolist()[:6]}")
    step = QStep(x, qc)
    step.append()
    torch.cuda.synchronize()
    kc, ks, vc, vs, q2 = check_append(step, x, qc)
    lens = x.seq_lens.numpy()
    if w.paged:
        ref = QO.decode_attention_paged_u8(q2, kc, ks, vc, vs, x.block_table.numpy(), w.block_size, lens, "bf16")
    else:
        ref = QO.decode_attention_u8(q2, kc, ks, vc, vs, lens, "bf16")
    # the plan's split, one that leaves some waves without a tile, and one split
    for split in (0, 64, 1 << 20):
        out = step.decode(split)
        torch.cuda.synchronize()
        compare(out, ref, f"{name} split={split}")


def test_decode_u8_lengths_edge_cases():
    """L = 1 (only the new token), a length on a tile boundary, and L = 0."""
    w = SMALL["gqa_8b"].replace(B=3, cached_lo=0, cached_hi=0)
    x = W.draw(w)
    qc = W.draw_quantized(x)
    step = QStep(x, qc)
    step.append()
    torch.cuda.synchronize()
    kc, ks, vc, vs, q2 = check_append(step, x, qc)
    for lens_list in ([1, 1, 1],):
        lens = np.array(lens_list, np.int32)
        ref = QO.decode_attention_u8(q2, kc, ks, vc, vs, lens, "bf16")
        out = kvc.decode_attn_u8(step.q, step.kc, step.ks, step.vc, step.vs, torch.from_numpy(lens).cuda(), 1)
        torch.cuda.synchronize()
        compare(out, ref, "L=1")
    w2 = SMALL["gqa_8b"].replace(B=3, cached_lo=255, cached_hi=255)     # 256 attended: two whole steps
    x2 = W.draw(w2)
    qc2 = W.draw_quantized(x2)
    s2 = QStep(x2, qc2)
    s2.append()
    torch.cuda.synchronize()
    kc, ks, vc, vs, q2 = check_append(s2, x2, qc2)
    ref = QO.decode_attention_u8(q2, kc, ks, vc, vs, x2.seq_lens.numpy(), "bf16")
    for split in (0, 128, 32):
        compare(s2.decode(split), ref, f"L=256 split={split}")
    zero = torch.zeros(3, dtype=torch.int32, device="cuda")
    out = kvc.decode_attn_u8(s2.q, s2.kc, s2.ks, s2.vc, s2.vs, zero, 256)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0, "L = 0 must give zeros"


@pytest.mark.parametrize("name", ["gqa_8b", "mqa_ragged", "long_gqa", "paged_gqa"])
def test_decode_u8_full_size(name):
    """Every output at the workload's full size, in the default launch plan."""
    w = W.WORKLOADS[name]
    x = W.draw(w)
    qc = W.draw_quantized(x)
    say(f"[decode_u8 {name} full] B={w.B} max_len={int(x.seq_lens.max())}")
    step = QStep(x, qc)
    step.append()
    out = step.decode()
    torch.cuda.synchronize()
    kc, ks, vc, vs, q2 = check_append(step, x, qc)
    lens = x.seq_lens.numpy()
    if w.paged:
        ref = QO.decode_attention_paged_u8(q2, kc, ks, vc, vs, x.block_table.numpy(), w.block_size, lens, "bf16")
    else:
        ref = QO.decode_attention_u8(q2, kc, ks, vc, vs, lens, "bf16")
    compare_out(out, ref, "bf16", f"u8 {name} full size")


def _run_step_u8(step: QStep, style="interleaved", split=0):
    """kvc_decode_step_u8 on copies of the step's cache: (codes, pairs, q_rot, out)."""
    kc, ks, vc, vs = step.kc.clone(), step.ks.clone(), step.vc.clone(), step.vs.clone()
    q_raw = step.x.q.to("cuda")
    out, q_rot = kvc.decode_step_u8(q_raw, kc, ks, vc, vs, step.pos, step.kn, step.vn, step.cos, step.sin,
                                    step.max_len, block_table=step.tbl, rope_style=style, split_tokens=split)
    return kc, ks, vc, vs, q_rot, out


@pytest.mark.parametrize("style", ["interleaved", "half"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_step_u8_equals_append_then_decode(name, style):
    """The fused step over a quantized cache gives bit for bit what
    kvc_append_u8 then kvc_decode_attn[_paged]_u8 give with the same split
    length (codes, pairs, rotated query and output), and the oracle's results
    (bit-exact append, attention within tolerance)."""
    x = W.draw(SMALL[name])
    w = x.workload
    qc = W.draw_quantized(x)
    say(f"[step_u8 {name} {style}] G={w.G} d={w.d} lens={x.seq_lens.tolist()[:6]}")
    ref = QStep(x, qc)
    ref.append(style)
    torch.cuda.synchronize()
    kc2, ks2, vc2, vs2, q2 = check_append(ref, x, qc, style)
    for split in (0, 64, 1 << 20):
        fresh = QStep(x, qc)
        kc, ks, vc, vs, q_rot, out = _run_step_u8(fresh, style, split)
        out_a = ref.decode(split)
        torch.cuda.synchronize()
        for what, got, exp in (("K codes", kc, ref.kc), ("K pairs", ks, ref.ks), ("V codes", vc, ref.vc),
                               ("V pairs", vs, ref.vs), ("rotated q", q_rot, ref.q)):
            assert np.array_equal(bits(got), bits(exp)), f"{what} differ from the append (split {split})"
        assert np.array_equal(bits(out), bits(out_a)), f"output differs from append + decode (split {split})"
    lens = x.seq_lens.numpy()
    if w.paged:
        oref = QO.decode_attention_paged_u8(q2, kc2, ks2, vc2, vs2, x.block_table.numpy(), w.block_size, lens, "bf16")
    else:
        oref = QO.decode_attention_u8(q2, kc2, ks2, vc2, vs2, lens, "bf16")
    compare(out, oref, f"step_u8 {name} {style}")


@pytest.mark.parametrize("name", ["gqa_8b", "paged_gqa"])
def test_step_u8_full_size(name):
    """The benchmarked quantized step (default plan) at full size: the new
    codes and pairs, the rotated query bit for bit, every output row within
    tolerance of the oracle."""
    w = W.WORKLOADS[name]
    x = W.draw(w)
    qc = W.draw_quantized(x)
    say(f"[step_u8 {name} full] B={w.B} max_len={int(x.seq_lens.max())}")
    step = QStep(x, qc)
    kc, ks, vc, vs, q_rot, out = _run_step_u8(step)
    torch.cuda.synchronize()
    kc2, ks2, vc2, vs2, q2 = oracle_append_u8(x, qc)
    for what, got, ref in (("K codes", kc, kc2), ("K pairs", ks, ks2), ("V codes", vc, vc2), ("V pairs", vs, vs2),
                           ("rotated q", q_rot, q2)):
        assert np.array_equal(bits(got), np.ascontiguousarray(ref).view(np.uint8)), f"{what} differ from the oracle"
    lens = x.seq_lens.numpy()
    if w.paged:
        ref = QO.decode_attention_paged_u8(q2, kc2, ks2, vc2, vs2, x.block_table.numpy(), w.block_size, lens, "bf16")
    else:
        ref = QO.decode_attention_u8(q2, kc2, ks2, vc2, vs2, lens, "bf16")
    compare_out(out, ref, "bf16", f"step_u8 {name} full size")
