"""Plain CPU oracle for a decode step over a quantized KV cache: uint8 codes with
one (scale, zero point) pair per cached vector.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module.  Like the unquantized oracle it has no
tiling, splitting or fusion; every function can be read against its source.

Source: [BLOG] "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리
효율화 전략" (youngju.dev), the QuantizedKVCache listing.  Per vector over the
last axis it takes the minimum and maximum, sets the step to (max - min) / 255
and the zero point to -min / step rounded and clamped to [0, 255], stores the
codes x / step + zero point rounded and clamped to [0, 255] as uint8, and reads
a cached value back as (code - zero point) * step in float32.  The listing keeps
a single (step, zero point) per update and replaces it on the next one, so the
older tokens could no longer be read back; here every cached vector keeps its
own pair, per (sequence, KV head, token), which is what reading them requires.

Readings (also listed in the design notes):
* The listing works on float tensors: every operation is float32, rounded once;
  "round" is to nearest with ties to even.
* The key is quantized after rotation, from its float32 rotated value (the
  rotation sequence of the unquantized oracle, before its storage rounding);
  the value from its input dtype converted to float32.
* A constant vector (max == min) gives a zero step, which the listing divides
  by; its step is taken as 1.
* A vector whose range does not contain 0 has its zero point clamped, and its
  codes clip at 255 (the listing as written); synthetic N(0, 1) vectors of the
  workloads always straddle 0.
* Attention is the plain definition of the unquantized oracle, in float64, over
  the dequantized float32 values.
* Cache layout: codes uint8 [B, H_kv, T, d] (contiguous) or [N_blk, H_kv, bs, d]
  (paged, as the unquantized pools); their (step, zero point) pairs float32
  [..., 2] with the same leading axes.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import kvc_oracle as O

__all__ = ["quantize_u8", "dequantize_u8", "append_contiguous_u8", "append_paged_u8",
           "decode_attention_u8", "decode_attention_paged_u8", "decode_kv_read_bytes_u8"]

# An 8-bit affine grid has 256 codes, so 255 steps between its end points.
_STEPS = np.float32(255.0)
_TOP_CODE = 255


def _affine_grid(lo: np.ndarray, hi: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Step and zero code of the 256-code grid whose end codes sit at the
    vector's extremes lo and hi (float32 arrays, one entry per vector).

    The step is the span over 255 steps; the zero code is the code nearest to
    the value 0, kept on the grid.  A vector with no span gets step 1 (the page
    divides by its zero step there).
    """
    step = (hi - lo) / _STEPS
    step = np.where(step == 0, np.float32(1.0), step).astype(np.float32)
    zero = np.clip(np.rint(np.negative(lo) / step), 0, _TOP_CODE).astype(np.float32)
    return step, zero


def _encode(x: np.ndarray, step: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """Code of each value: its distance from the zero code in steps, rounded
    to the nearest code (ties to even) and kept on the grid."""
    return np.clip(np.rint(x / step + zero), 0, _TOP_CODE).astype(np.uint8)


def quantize_u8(x) -> Tuple[np.ndarray, np.ndarray]:
    """uint8 codes and float32 [..., 2] (step, zero point) pairs of the vectors
    along the last axis of x.  Every operation is one float32 operation,
    rounded once (the precision the page's float tensors have)."""
    v = np.asarray(x, dtype=np.float32)
    step, zero = _affine_grid(np.min(v, axis=-1, keepdims=True), np.max(v, axis=-1, keepdims=True))
    return _encode(v, step, zero), np.concatenate([step, zero], axis=-1).astype(np.float32)


def dequantize_u8(codes, sz) -> np.ndarray:
    """float32 values (code - zero point) * step of cached vectors."""
    sz = np.asarray(sz, dtype=np.float32)
    step, zp = sz[..., 0:1], sz[..., 1:2]
    return (np.asarray(codes).astype(np.float32) - zp) * step


def _quantized_kv(k_new, v_new, p, cos, sin, dtype, style):
    """Codes and pairs of sequence b's new key (rotated at p) and value, [H_kv, d]."""
    kr = O.rope_rotate_f32(k_new, dtype, cos[p], sin[p], style).astype(np.float32)
    return quantize_u8(kr), quantize_u8(O.to_f32(v_new, dtype))


def append_contiguous_u8(k_codes, k_sz, v_codes, v_sz, cached, k_new, v_new, cos, sin, dtype,
                         style="interleaved", q=None):
    """Quantize rotated k_new and raw v_new into slot cached[b] of the code and
    pair arrays; q (if given) is rotated at the same position as in the
    unquantized oracle.  Returns new arrays; nothing else changes."""
    kc, ks, vc, vs = (np.array(a, copy=True) for a in (k_codes, k_sz, v_codes, v_sz))
    q2 = None if q is None else np.array(q, copy=True)
    for b, p in enumerate(np.asarray(cached).tolist()):
        (ck, sk), (cv, sv) = _quantized_kv(k_new[b], v_new[b], p, cos, sin, dtype, style)
        kc[b, :, p, :], ks[b, :, p, :] = ck, sk
        vc[b, :, p, :], vs[b, :, p, :] = cv, sv
        if q2 is not None:
            q2[b] = O.rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return kc, ks, vc, vs, q2


def append_paged_u8(k_codes, k_sz, v_codes, v_sz, block_table, block_size, cached, k_new, v_new,
                    cos, sin, dtype, style="interleaved", q=None):
    """Paged form: the slot of position p is [table[b][p // bs], :, p % bs]."""
    kc, ks, vc, vs = (np.array(a, copy=True) for a in (k_codes, k_sz, v_codes, v_sz))
    q2 = None if q is None else np.array(q, copy=True)
    for b, p in enumerate(np.asarray(cached).tolist()):
        lb, off = O.paged_location(p, block_size)
        phys = int(block_table[b][lb])
        (ck, sk), (cv, sv) = _quantized_kv(k_new[b], v_new[b], p, cos, sin, dtype, style)
        kc[phys, :, off, :], ks[phys, :, off, :] = ck, sk
        vc[phys, :, off, :], vs[phys, :, off, :] = cv, sv
        if q2 is not None:
            q2[b] = O.rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return kc, ks, vc, vs, q2


def decode_attention_u8(q, k_codes, k_sz, v_codes, v_sz, seq_lens, dtype, scale: Optional[float] = None):
    """Float64 output [B, H_q, d]: the unquantized definition over the
    dequantized first L_b vectors of each group's cache."""
    B = q.shape[0]
    k = np.zeros(k_codes.shape, np.float32)
    v = np.zeros(v_codes.shape, np.float32)
    for b in range(B):
        L = int(seq_lens[b])
        k[b, :, :L] = dequantize_u8(k_codes[b, :, :L], k_sz[b, :, :L])
        v[b, :, :L] = dequantize_u8(v_codes[b, :, :L], v_sz[b, :, :L])
    return _decode_f32_cache(q, k, v, seq_lens, dtype, scale)


def _decode_f32_cache(q, k, v, seq_lens, dtype, scale):
    """q in its storage dtype, dequantized cache in float32: the unquantized
    definition with each operand converted exactly to float64."""
    B, H_q, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    qf = O.to_f64(q, dtype)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(H_kv):
            K = k[b, j, :L].astype(np.float64)
            V = v[b, j, :L].astype(np.float64)
            for h in range(j * G, (j + 1) * G):
                out[b, h], _ = O._head_attention(qf[b, h], K, V, sc)
    return out


def decode_attention_paged_u8(q, k_codes, k_sz, v_codes, v_sz, block_table, block_size, seq_lens,
                              dtype, scale: Optional[float] = None):
    """Paged cache: gather each sequence's codes and pairs, then the contiguous form."""
    B = q.shape[0]
    H_kv, d = k_codes.shape[1], k_codes.shape[3]
    Lmax = max(int(L) for L in seq_lens) if B else 0
    kc = np.zeros((B, H_kv, Lmax, d), np.uint8)
    vc = np.zeros((B, H_kv, Lmax, d), np.uint8)
    ks = np.zeros((B, H_kv, Lmax, 2), np.float32)
    vs = np.zeros((B, H_kv, Lmax, 2), np.float32)
    for b in range(B):
        L = int(seq_lens[b])
        kc[b, :, :L] = O.gather_paged(k_codes, block_table, block_size, b, L)
        vc[b, :, :L] = O.gather_paged(v_codes, block_table, block_size, b, L)
        ks[b, :, :L] = O.gather_paged(k_sz, block_table, block_size, b, L)
        vs[b, :, :L] = O.gather_paged(v_sz, block_table, block_size, b, L)
    return decode_attention_u8(q, kc, ks, vc, vs, seq_lens, dtype, scale)


def decode_kv_read_bytes_u8(seq_lens, H_kv: int, d: int) -> int:
    """Bytes of the quantized cache one decode step reads: per token and KV head
    d codes and one 8-byte pair, for K and for V."""
    return int(sum(int(L) for L in seq_lens)) * H_kv * (d + 8) * 2
