"""GPU parity of the latent-cache decode (kvc_append_mla, kvc_decode_attn_mla,
kvc_decode_step_mla) against the MLA oracle, through the C ABI.

The oracle follows the MultiHeadLatentAttention listing of "KV Cache 최적화
심층 분석" (youngju.dev) as written: keys and values up-projected per head from
the cached latents, then the plain softmax attention in float64.  The GPU
computes the absorbed form.  Bars: the append is bit-exact over the whole
cache; the float32 output is within 2e-3 (max abs) of the float64 oracle.
"""
import numpy as np
import pytest
import torch

import mqa_decode_attention_amd as kvc
import oracle.kvc_mla_oracle as MLA
import workloads as W
from gpu_helpers import bits, say, store_np

pytestmark = pytest.mark.gpu

TOL = 2e-3
BASE = W.MLA_WORKLOADS["mla_latent"]


def _case(B, H, d_k, dl, rd, lo, hi, T_max=None, seed=101):
    w = BASE.replace(seed=seed, B=B, H=H, d_k=d_k, d_latent=dl, rope_dim=rd, cached_lo=lo, cached_hi=hi,
                     T_max=T_max or -(-(hi + 1) // 8) * 8)
    return w, W.draw_mla(w)


def _np(x: W.MlaInputs):
    dt = x.workload.dtype
    return {k: store_np(getattr(x, k), dt) for k in ("cache", "q", "c_kv_new", "k_rope_new", "w_uk", "b_uk",
                                                     "w_uv", "b_uv")}


def _oracle_step(x: W.MlaInputs):
    """Cache after the append and the float64 output over L = cached + 1."""
    n = _np(x)
    w = x.workload
    c2 = MLA.append_mla(n["cache"], x.cached.numpy(), n["c_kv_new"], n["k_rope_new"])
    o = MLA.decode_attention_mla(n["q"], c2, x.seq_lens.numpy(), n["w_uk"], n["b_uk"], n["w_uv"], n["b_uv"],
                                 w.d_latent, w.dtype)
    return c2, o


class Dev:
    def __init__(self, x: W.MlaInputs):
        self.x = x
        for k in ("cache", "q", "c_kv_new", "k_rope_new", "w_uk", "w_uv", "b_uv"):
            setattr(self, k, getattr(x, k).cuda())
        self.pos = x.cached.cuda()
        self.lens = x.seq_lens.cuda()
        self.max_len = int(x.seq_lens.max())

    def append(self, cache=None):
        c = self.cache if cache is None else cache
        kvc.append_mla(c, self.pos, self.c_kv_new, self.k_rope_new if self.x.workload.rope_dim else None)
        return c

    def decode(self, cache=None, lens=None, max_len=None, split_tokens=0, b_uv=True):
        return kvc.decode_attn_mla(self.q, self.cache if cache is None else cache,
                                   self.lens if lens is None else lens,
                                   self.max_len if max_len is None else max_len, self.w_uk, self.w_uv,
                                   self.b_uv if b_uv else None, split_tokens=split_tokens)

    def step(self, split_tokens=0):
        c = self.cache.clone()
        out = kvc.decode_step_mla(self.q, c, self.pos, self.c_kv_new,
                                  self.k_rope_new if self.x.workload.rope_dim else None, self.max_len,
                                  self.w_uk, self.w_uv, self.b_uv, split_tokens=split_tokens)
        return c, out


def _bytes(t: torch.Tensor) -> np.ndarray:
    return bits(t).reshape(-1)


def _bytes_np(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def _compare(got: torch.Tensor, ref: np.ndarray, what: str):
    g = got.detach().cpu().double().numpy()
    assert g.shape == ref.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    say(f"  {what}: max|err| = {err:.3g} (tol {TOL}), max|out| = {float(np.max(np.abs(ref))):.3g}")
    assert err <= TOL, f"{what}: max abs error {err} > {TOL}"


# (B, H, d_k, d_latent, rope_dim, cached lo, cached hi)
SHAPES = [
    (3, 32, 128, 512, 64, 0, 300),     # the workload's heads and widths, ragged lengths
    (2, 16, 64, 256, 0, 40, 200),      # one 16-head block, no rope part
    (2, 8, 32, 128, 8, 100, 130),      # narrow latent, 8 heads
    (2, 40, 64, 512, 64, 60, 150),     # two head chunks (32 + 8)
    (2, 64, 128, 512, 64, 90, 140),    # two full chunks
    (19, 32, 128, 512, 64, 0, 70),     # more than 16 sequences in the up-projections
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_H{}_dk{}_dl{}_rd{}_L{}-{}".format(*s))
def test_append_and_decode(shape):
    B, H, d_k, dl, rd, lo, hi = shape
    w, x = _case(B, H, d_k, dl, rd, lo, hi)
    say(f"mla case {w}")
    c2, ref = _oracle_step(x)
    d = Dev(x)
    d.append()
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(d.cache), _bytes_np(c2)), "append differs"
    for split in (0, 32, 64, 256):
        out = d.decode(split_tokens=split)
        torch.cuda.synchronize()
        _compare(out, ref, f"split {split} (plan {kvc.mla_split_tokens(B, H, dl, d.max_len, split)})")


def test_edge_lengths():
    """L = 0 gives zeros; L = 1 gives W_uv c_0 + b_uv; lengths on tile and split
    boundaries; max_seq_len = T_max."""
    w, x = _case(5, 32, 128, 512, 64, 255, 255, T_max=256, seed=103)
    c2, _ = _oracle_step(x)
    d = Dev(x)
    d.append()
    n = _np(x)
    lens = np.array([0, 1, 32, 64, 256], dtype=np.int32)
    ref = MLA.decode_attention_mla(n["q"], c2, lens, n["w_uk"], n["b_uk"], n["w_uv"], n["b_uv"], 512, "bf16")
    assert np.all(ref[0] == 0.0)
    lt = torch.from_numpy(lens).cuda()
    for split in (0, 32, 64):
        out = d.decode(lens=lt, max_len=256, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.all(out[0] == 0), "a sequence of length 0 must give zeros"
        _compare(out, ref, f"edge lengths, split {split}")


def test_without_value_bias():
    w, x = _case(2, 32, 128, 512, 64, 10, 90, seed=104)
    c2, _ = _oracle_step(x)
    n = _np(x)
    zero = np.zeros_like(n["b_uv"])
    ref = MLA.decode_attention_mla(n["q"], c2, x.seq_lens.numpy(), n["w_uk"], n["b_uk"], n["w_uv"], zero, 512,
                                   "bf16")
    d = Dev(x)
    d.append()
    out = d.decode(b_uv=False)
    torch.cuda.synchronize()
    _compare(out, ref, "b_uv = NULL")


def test_step_equals_append_then_decode_and_oracle():
    w, x = _case(4, 32, 128, 512, 64, 1, 400, seed=105)
    c2, ref = _oracle_step(x)
    d = Dev(x)
    for split in (0, 64):
        cs, out_s = d.step(split_tokens=split)
        c = d.cache.clone()
        d.append(c)
        out_a = kvc.decode_attn_mla(d.q, c, d.lens, d.max_len, d.w_uk, d.w_uv, d.b_uv, split_tokens=split)
        torch.cuda.synchronize()
        assert np.array_equal(_bytes(cs), _bytes_np(c2)), "step append differs"
        assert torch.equal(out_s, out_a), "step != append + decode"
        _compare(out_s, ref, f"step, split {split}")


def test_deterministic_and_workspace_reuse():
    w, x = _case(3, 32, 128, 512, 64, 200, 500, seed=106)
    d = Dev(x)
    d.append()
    B, H, dl = w.B, w.H, w.d_latent
    need = kvc.mla_workspace_bytes(B, H, dl, d.max_len, 64)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # garbage (NaN patterns) in the workspace
    a = kvc.decode_attn_mla(d.q, d.cache, d.lens, d.max_len, d.w_uk, d.w_uv, d.b_uv, split_tokens=64,
                            workspace=ws)
    b = kvc.decode_attn_mla(d.q, d.cache, d.lens, d.max_len, d.w_uk, d.w_uv, d.b_uv, split_tokens=64,
                            workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_size():
    """The latent workload at full size (16 sequences of 8192 cached tokens,
    32 heads of 128, d_latent 512, rope 64) through the decode step in the
    launch configuration the benchmark times: the appended rows bit for bit,
    and every output against the listing as written (which up-projects each
    sequence's whole cache for all heads, about 70 GFLOP of float64 per
    sequence on the host)."""
    x = W.draw_mla(BASE)
    d = Dev(x)
    say(f"full size {BASE.name}: split {kvc.mla_split_tokens(BASE.B, BASE.H, BASE.d_latent, d.max_len)}")
    c, out = d.step()
    torch.cuda.synchronize()
    n = _np(x)
    pos = x.cached.numpy()
    cg = c.cpu()
    for b in range(BASE.B):
        row = store_np(cg[b, pos[b]], "bf16")
        assert np.array_equal(row, np.concatenate([n["c_kv_new"][b], n["k_rope_new"][b]])), f"row of sequence {b}"
    c2 = MLA.append_mla(n["cache"], pos, n["c_kv_new"], n["k_rope_new"])
    ref = MLA.decode_attention_mla(n["q"], c2, x.seq_lens.numpy(), n["w_uk"], n["b_uk"], n["w_uv"], n["b_uv"],
                                   BASE.d_latent, "bf16")
    _compare(out, ref, "full size, every output")
