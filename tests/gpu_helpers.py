"""Shared steps of the GPU tests: run the HIP path, run the oracle, compare.

The GPU side goes through the Python binding (and so the C ABI); the oracle
side sees the same seeded inputs and never anything the GPU produced.
"""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

import mqa_decode_attention_amd as kvc
import oracle as O
import workloads as W

BF16_TOL = 2e-3      # max-abs bar for bf16 attention outputs (after bf16 rounding of the oracle)
F32_TOL = 1e-5       # float32 outputs: far inside the same bar
# Half-width of the band around a bf16 rounding midpoint inside which both
# neighbouring bf16 values are correct results of a float32-accumulated
# computation: the kernels' float32 results lie within ~1e-6 of the exact
# value for outputs of order 1 (weights carried to ~24 bits, float32 sums), so
# an exact value this close to a midpoint may round either way.  Above
# |O| = 0.5 one bf16 step (3.9e-3) exceeds the 2e-3 bar, so such a tie would
# otherwise fail whichever way a correct computation rounds.
BF16_TIE_BAND = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def store_np(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


class GpuStep:
    """Inputs on the GPU, the append and the decode call, results back on the CPU."""

    def __init__(self, x: W.DecodeInputs, device: str = "cuda"):
        self.x = x
        w = x.workload
        self.k = x.k_cache.to(device)
        self.v = x.v_cache.to(device)
        self.q = x.q.to(device).clone()
        self.kn = x.k_new.to(device)
        self.vn = x.v_new.to(device)
        self.pos = x.cached.to(device)
        self.lens = x.seq_lens.to(device)
        self.cos = x.rope_cos.to(device)
        self.sin = x.rope_sin.to(device)
        self.tbl = x.block_table.to(device) if w.paged else None
        self.max_len = int(x.seq_lens.max())

    def append(self, rope_style="interleaved", stream=None):
        kvc.append(self.k, self.v, self.pos, self.kn, self.vn, self.cos, self.sin, q=self.q,
                   block_table=self.tbl, rope_style=rope_style, stream=stream)

    def decode(self, split_tokens=0, lens=None, max_len=None, stream=None, out=None):
        lens = self.lens if lens is None else lens
        max_len = self.max_len if max_len is None else max_len
        if self.tbl is not None:
            return kvc.decode_attn_paged(self.q, self.k, self.v, self.tbl, lens, max_len,
                                         split_tokens=split_tokens, stream=stream, out=out)
        return kvc.decode_attn(self.q, self.k, self.v, lens, max_len, split_tokens=split_tokens,
                               stream=stream, out=out)


def oracle_append(x: W.DecodeInputs, rope_style="interleaved"):
    """Oracle caches and rotated q after the append (numpy storage arrays)."""
    w = x.workload
    dt = w.dtype
    kc, vc = store_np(x.k_cache, dt), store_np(x.v_cache, dt)
    q, kn, vn = store_np(x.q, dt), store_np(x.k_new, dt), store_np(x.v_new, dt)
    cos, sin = x.rope_cos.numpy(), x.rope_sin.numpy()
    cached = x.cached.numpy()
    if w.paged:
        return O.append_paged(kc, vc, x.block_table.numpy(), w.block_size, cached, kn, vn, cos, sin,
                              dt, rope_style, q=q)
    return O.append_contiguous(kc, vc, cached, kn, vn, cos, sin, dt, rope_style, q=q)


def oracle_decode(x: W.DecodeInputs, k2, v2, q2, seq_lens=None):
    w = x.workload
    lens = x.seq_lens.numpy() if seq_lens is None else seq_lens
    if w.paged:
        o = O.decode_attention_paged(q2, k2, v2, x.block_table.numpy(), w.block_size, lens, w.dtype)
    else:
        o = O.decode_attention(q2, k2, v2, lens, w.dtype)
    return o


def ulp_distance(a: np.ndarray, b: np.ndarray, dtype: str) -> int:
    """Largest distance, in units in the last place of the storage dtype,
    between two arrays of stored values (bit patterns mapped onto a signed
    integer line, so neighbouring representable values are 1 apart)."""
    if a.size == 0:
        return 0
    ut, st, top = (np.uint16, np.int64, 0x8000) if dtype == "bf16" else (np.uint32, np.int64, 0x80000000)

    def line(x):
        u = np.ascontiguousarray(x).view(ut).astype(st)
        return np.where(u & top, -(u & (top - 1)), u)

    return int(np.max(np.abs(line(a) - line(b))))


def _ulp_steps(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Elementwise distance in storage-dtype ulps (see ulp_distance)."""
    ut, top = (np.uint16, 0x8000) if dtype == "bf16" else (np.uint32, 0x80000000)

    def line(x):
        u = np.ascontiguousarray(x).view(ut).astype(np.int64)
        return np.where(u & top, -(u & (top - 1)), u)

    return np.abs(line(a) - line(b))


def compare_out(got: torch.Tensor, ref64: np.ndarray, dtype: str, what: str = ""):
    """Max-abs error of the GPU output against the oracle rounded to the storage
    dtype, over every output; also reports max|out| and the largest distance in
    storage-dtype ulps, so the headroom under the bar is visible.

    bf16 outputs whose exact (float64) value lies within BF16_TIE_BAND of the
    midpoint between two bf16 values have two correct results: the GPU value
    may be either neighbour there (counted and reported as ties, and excluded
    from max|err|); every other output must be within the bar."""
    gs = store_np(got, dtype)
    rs = O.round_store(ref64, dtype)
    g = O.to_f64(gs, dtype)
    r = O.to_f64(rs, dtype)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    e = np.abs(g - r)
    ties = np.zeros(e.shape, dtype=bool)
    if dtype == "bf16" and g.size:
        mid = 0.5 * (g + r)
        ties = (e > tol) & (_ulp_steps(gs, rs, dtype) == 1) & \
            (np.abs(np.asarray(ref64, np.float64).reshape(g.shape) - mid) <= BF16_TIE_BAND)
    err = float(np.max(np.where(ties, 0.0, e))) if g.size else 0.0
    say(f"  {what}: {g.size} outputs, max|err| = {err:.3g} (tol {tol}), "
        f"max|out| = {float(np.max(np.abs(r))) if r.size else 0:.3g}, max ulp distance = {ulp_distance(gs, rs, dtype)}"
        + (f", rounding ties taken the other way: {int(ties.sum())}" if ties.any() else ""))
    assert err <= tol, f"{what}: max abs error {err} > {tol}"
    return err


def run_step(step: "GpuStep", split_tokens=0, rope_style="interleaved", stream=None):
    """kvc_decode_step on fresh copies of the step's inputs: (k, v, q_rot, out)."""
    x = step.x
    k, v = step.k.clone(), step.v.clone()
    q_raw = x.q.to(step.k.device)
    out, q_rot = kvc.decode_step(q_raw, k, v, step.pos, step.kn, step.vn, step.cos, step.sin,
                                 step.max_len, block_table=step.tbl, rope_style=rope_style,
                                 split_tokens=split_tokens, stream=stream)
    return k, v, q_rot, out
