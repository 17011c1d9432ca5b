"""GPU parity of the FP8 cache path (E4M3 codes with a float32 scale per cached
vector, or E5M2 codes with scale 1) with its oracle, through the C ABI.

* Every finite code of each format must read back exactly as the oracle's
  decoding table gives it (one attended token with scale 1: the output is the
  value row itself, exact in bf16).
* kvc_append_fp8 must give the oracle's codes, pairs and rotated query bit for
  bit (codes decided in float32 by both sides, round to nearest even).
* kvc_decode_attn[_paged]_fp8 must match the oracle's float64 attention over
  the dequantized values within 2e-3 after bf16 rounding, for several splits,
  both layouts, head_dim 64 and 128, groups of 4 to 32 heads.
* kvc_decode_step_fp8 must equal append + decode bit for bit, and at the
  workloads' full sizes (gqa_8b, paged_gqa) match the oracle on every output.

Inputs: the workloads' seeded draws for the queries and new tokens, and FP8
caches drawn by workloads.draw_fp8.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import oracle.kvc_fp8_oracle as FO
import workloads as W
from gpu_helpers import bits, compare_out, say, store_np

pytestmark = pytest.mark.gpu

FMTS = ("e4m3", "e5m2")
SMALL = {
    "gqa_8b": W.WORKLOADS["gqa_8b"].replace(B=3, cached_lo=300, cached_hi=1100, T_max=1104),
    "mqa_ragged": W.WORKLOADS["mqa_ragged"].replace(B=5, cached_lo=100, cached_hi=700, T_max=704),
    "paged_gqa": W.WORKLOADS["paged_gqa"].replace(B=4, cached_lo=20, cached_hi=400),
    "gqa_d64": W.WORKLOADS["gqa_8b"].replace(B=2, d=64, cached_lo=150, cached_hi=500, T_max=504),
    "paged_mqa": W.WORKLOADS["paged_gqa"].replace(B=3, H_q=24, H_kv=1, cached_lo=50, cached_hi=300),
}


class FStep:
    def __init__(self, x: W.DecodeInputs, qc: W.QuantCache, fmt: str, device="cuda"):
        w = x.workload
        self.x, self.fmt = x, fmt
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
        kvc.append_fp8(self.kc, self.ks, self.vc, self.vs, self.pos, self.kn, self.vn, self.cos, self.sin,
                       q=self.q, block_table=self.tbl, rope_style=style, fmt=self.fmt)

    def decode(self, split_tokens=0):
        if self.tbl is not None:
            return kvc.decode_attn_paged_fp8(self.q, self.kc, self.ks, self.vc, self.vs, self.tbl, self.lens,
                                             self.max_len, split_tokens=split_tokens, fmt=self.fmt)
        return kvc.decode_attn_fp8(self.q, self.kc, self.ks, self.vc, self.vs, self.lens, self.max_len,
                                   split_tokens=split_tokens, fmt=self.fmt)


def oracle_append(x, qc, fmt, style="interleaved"):
    w = x.workload
    dt = w.dtype
    arrs = (qc.k_codes.numpy(), qc.k_sz.numpy(), qc.v_codes.numpy(), qc.v_sz.numpy())
    q, kn, vn = store_np(x.q, dt), store_np(x.k_new, dt), store_np(x.v_new, dt)
    cos, sin = x.rope_cos.numpy(), x.rope_sin.numpy()
    cached = x.cached.numpy()
    if w.paged:
        return FO.append_paged_fp8(*arrs, x.block_table.numpy(), w.block_size, cached, kn, vn, cos, sin, dt, fmt,
                                   style, q=q)
    return FO.append_contiguous_fp8(*arrs, cached, kn, vn, cos, sin, dt, fmt, style, q=q)


def oracle_decode(x, arrs, q2, fmt):
    w = x.workload
    kc, ks, vc, vs = arrs
    lens = x.seq_lens.numpy()
    if w.paged:
        return FO.decode_attention_paged_fp8(q2, kc, ks, vc, vs, x.block_table.numpy(), w.block_size, lens, "bf16",
                                             fmt)
    return FO.decode_attention_fp8(q2, kc, ks, vc, vs, lens, "bf16", fmt)


def check_append(step: FStep, x, qc, style="interleaved"):
    kc, ks, vc, vs, q2 = oracle_append(x, qc, step.fmt, style)
    for name, got, ref in (("K codes", step.kc, kc), ("K pairs", step.ks, ks), ("V codes", step.vc, vc),
                           ("V pairs", step.vs, vs)):
        assert np.array_equal(bits(got), np.ascontiguousarray(ref).view(np.uint8)), f"{name} differ from the oracle"
    assert np.array_equal(store_np(step.q, x.workload.dtype).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8)), \
        "rotated q differs from the oracle"
    return (kc, ks, vc, vs), q2


@pytest.mark.parametrize("fmt", FMTS)
def test_every_code_reads_back_exactly(fmt):
    """One attended token whose value row holds every finite code (scale 1):
    each output is that code's value, exactly."""
    table = FO.fp8_table(fmt)
    finite = [c for c in range(256) if np.isfinite(table[c])]
    B, H_q, H_kv, d = 2, 2, 2, 128
    vals = np.array((finite * 4)[:B * H_kv * d], np.uint8).reshape(B, H_kv, d)
    w = W.WORKLOADS["gqa_8b"].replace(B=B, H_q=H_q, H_kv=H_kv, cached_lo=3, cached_hi=3, T_max=8)
    x = W.draw(w)
    qc = W.draw_fp8(x, fmt)
    qc.v_codes[:, :, 0, :] = torch.from_numpy(vals)
    qc.v_sz[:, :, 0, :] = torch.tensor([1.0, 0.0])
    qc.k_sz[:, :, 0, :] = torch.tensor([1.0, 0.0])
    step = FStep(x, qc, fmt)
    ones = torch.ones(B, dtype=torch.int32, device="cuda")
    out = kvc.decode_attn_fp8(step.q, step.kc, step.ks, step.vc, step.vs, ones, 1, fmt=fmt)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy().astype(np.float64).reshape(B, H_q, d)
    want = table[vals.reshape(B, H_kv, d)]           # G = 1: head h reads KV head h
    assert np.array_equal(g, want), f"{fmt}: codes read back wrong: {np.argwhere(g != want)[:4].tolist()}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", sorted(SMALL))
def test_append_fp8_bit_exact(name, fmt):
    x = W.draw(SMALL[name])
    qc = W.draw_fp8(x, fmt)
    say(f"[append_fp8 {fmt} {name}] lens={x.seq_lens.tolist()[:6]}")
    step = FStep(x, qc, fmt)
    step.append()
    torch.cuda.synchronize()
    check_append(step, x, qc)


@pytest.mark.parametrize("fmt", FMTS)
def test_append_fp8_half_rotation(fmt):
    x = W.draw(SMALL["gqa_8b"])
    qc = W.draw_fp8(x, fmt)
    step = FStep(x, qc, fmt)
    step.append("half")
    torch.cuda.synchronize()
    check_append(step, x, qc, "half")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_fp8_matches_oracle(name, fmt):
    x = W.draw(SMALL[name])
    w = x.workload
    qc = W.draw_fp8(x, fmt)
    say(f"[decode_fp8 {fmt} {name}] G={w.G} d={w.d} lens={x.seq_lens.tolist()[:6]}")
    step = FStep(x, qc, fmt)
    step.append()
    torch.cuda.synchronize()
    arrs, q2 = check_append(step, x, qc)
    ref = oracle_decode(x, arrs, q2, fmt)
    for split in (0, 64, 1 << 20):
        out = step.decode(split)
        torch.cuda.synchronize()
        compare_out(out, ref, "bf16", f"{fmt} {name} split={split}")


def _run_step(step: FStep, style="interleaved", split=0):
    """kvc_decode_step_fp8 on copies of the step's cache: (codes, pairs, q_rot, out)."""
    kc, ks, vc, vs = step.kc.clone(), step.ks.clone(), step.vc.clone(), step.vs.clone()
    q_raw = step.x.q.to("cuda")
    out, q_rot = kvc.decode_step_fp8(q_raw, kc, ks, vc, vs, step.pos, step.kn, step.vn, step.cos, step.sin,
                                     step.max_len, block_table=step.tbl, rope_style=style, split_tokens=split,
                                     fmt=step.fmt)
    return kc, ks, vc, vs, q_rot, out


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["gqa_8b", "mqa_ragged", "paged_gqa", "gqa_d64"])
def test_step_fp8_equals_append_then_decode(name, fmt):
    """The fused step (new key and value quantized inside the streaming kernel)
    gives bit for bit what the append then the decode give with the same
    split length, and the oracle's results."""
    x = W.draw(SMALL[name])
    qc = W.draw_fp8(x, fmt)
    say(f"[step_fp8 {fmt} {name}] lens={x.seq_lens.tolist()[:6]}")
    ref = FStep(x, qc, fmt)
    ref.append()
    torch.cuda.synchronize()
    arrs, q2 = check_append(ref, x, qc)
    for split in (0, 64, 1 << 20):
        kc, ks, vc, vs, q_rot, out = _run_step(FStep(x, qc, fmt), split=split)
        out_a = ref.decode(split)
        torch.cuda.synchronize()
        for what, got, exp in (("K codes", kc, ref.kc), ("K pairs", ks, ref.ks), ("V codes", vc, ref.vc),
                               ("V pairs", vs, ref.vs), ("rotated q", q_rot, ref.q)):
            assert np.array_equal(bits(got), bits(exp)), f"{what} differ from the append (split {split})"
        assert np.array_equal(bits(out), bits(out_a)), f"output differs from append + decode (split {split})"
    compare_out(out, oracle_decode(x, arrs, q2, fmt), "bf16", f"step_fp8 {fmt} {name}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["gqa_8b", "paged_gqa"])
def test_step_fp8_full_size(name, fmt):
    """The benchmarked FP8 step (default plan) at full size: the new codes and
    pairs and the rotated query bit for bit, every output within tolerance."""
    w = W.WORKLOADS[name]
    x = W.draw(w)
    qc = W.draw_fp8(x, fmt)
    say(f"[step_fp8 {fmt} {name} full] B={w.B} max_len={int(x.seq_lens.max())}")
    step = FStep(x, qc, fmt)
    kc, ks, vc, vs, q_rot, out = _run_step(step)
    torch.cuda.synchronize()
    kc2, ks2, vc2, vs2, q2 = oracle_append(x, qc, fmt)
    for what, got, ref in (("K codes", kc, kc2), ("K pairs", ks, ks2), ("V codes", vc, vc2), ("V pairs", vs, vs2),
                           ("rotated q", q_rot, q2)):
        assert np.array_equal(bits(got), np.ascontiguousarray(ref).view(np.uint8)), f"{what} differ from the oracle"
    compare_out(out, oracle_decode(x, (kc2, ks2, vc2, vs2), q2, fmt), "bf16", f"step_fp8 {fmt} {name} full size")


def _edge_vectors(fmt, d, rows):
    """bf16 vectors whose float32 values sit on the encoder's edge cases: the
    largest finite value first (an E4M3 vector's scale is then exactly 1, or
    3 for the second row: every element a tie after the division), then every
    midpoint between neighbouring values of the format (ties to even),
    subnormal ones included, alternating in sign; E5M2 rows end with a value
    past the largest finite one (saturation)."""
    table = FO.fp8_table(fmt)
    fin = np.sort(np.unique(np.abs(table[np.isfinite(table)])))
    mids = (fin[1:] + fin[:-1]) / 2
    vmax = fin[-1]
    out = np.zeros((rows, d), np.float64)
    for r in range(rows):
        s = 3.0 if (fmt == "e4m3" and r % 2 == 1) else 1.0
        v = np.concatenate([[vmax], np.roll(mids, 17 * r)])[:d]
        v = np.concatenate([v, np.zeros(max(0, d - v.size))])
        v[1::2] *= -1.0
        if fmt == "e5m2":
            v[-1] = 61440.0 * (-1.0 if r % 2 else 1.0)
        out[r] = v * s
    t = torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.double().numpy(), out), "edge values must be exact in bf16"
    return t


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_ties_subnormals_saturation(fmt):
    """The device encoder (append kernel and the fused step's own) on ties,
    subnormals and saturation, bit for bit against the oracle: new tokens at
    position 0, where the rotation is the identity."""
    B, H_q, H_kv, d = 2, 8, 2, 128
    w = W.WORKLOADS["gqa_8b"].replace(B=B, H_q=H_q, H_kv=H_kv, cached_lo=0, cached_hi=0, T_max=8)
    x = W.draw(w)
    x.k_new[:] = _edge_vectors(fmt, d, B * H_kv).reshape(B, H_kv, d)
    x.v_new[:] = _edge_vectors(fmt, d, B * H_kv).flip(0).reshape(B, H_kv, d)
    qc = W.draw_fp8(x, fmt)
    kc2, ks2, vc2, vs2, q2 = oracle_append(x, qc, fmt)
    # the append kernel
    step = FStep(x, qc, fmt)
    step.append()
    torch.cuda.synchronize()
    for what, got, ref in (("K codes", step.kc, kc2), ("K pairs", step.ks, ks2), ("V codes", step.vc, vc2),
                           ("V pairs", step.vs, vs2)):
        assert np.array_equal(bits(got), np.ascontiguousarray(ref).view(np.uint8)), f"append: {what} differ"
    # the fused step's encoder
    kc, ks, vc, vs, q_rot, out = _run_step(FStep(x, qc, fmt))
    torch.cuda.synchronize()
    for what, got, ref in (("K codes", kc, kc2), ("K pairs", ks, ks2), ("V codes", vc, vc2), ("V pairs", vs, vs2)):
        assert np.array_equal(bits(got), np.ascontiguousarray(ref).view(np.uint8)), f"fused step: {what} differ"
    # (sanity of the construction: ties and saturation were present)
    table = FO.fp8_table(fmt)
    assert np.any(np.abs(table[kc2[:, :, 0]]) == table[0x7E if fmt == "e4m3" else 0x7B])
