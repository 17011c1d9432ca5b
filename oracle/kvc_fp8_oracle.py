"""Plain CPU oracle for a decode step over an FP8 KV cache: one byte per cached
element in an 8-bit floating-point format, with one float32 scale per cached
vector.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module.  Like the other oracles it has no tiling,
splitting or fusion; every function can be read against its definition.

Sources.  "Arsitektur Inferensi LLM: PagedAttention, KV-Cache & Speculative
Decoding" (tveniu.com), section 2, sizes a GQA-8 cache quantized to FP8 or
INT8 at one byte per element, and its section 8 starts an engine with an "fp8"
KV-cache dtype; "KV Cache 최적화 심층 분석" (youngju.dev) turns on an fp8_e5m2
KV cache in its vLLM commands.  The pages fix the byte per element and name the
two formats; the rest is the reading below (also listed in the design notes).

Readings:
* Formats (the OCP 8-bit floating-point formats those names refer to):
  E4M3 - sign, 4 exponent bits (bias 7), 3 mantissa bits; subnormals below
  2^-6; no infinities, the codes S.1111.111 are NaN; largest finite 448.
  E5M2 - sign, 5 exponent bits (bias 15), 2 mantissa bits; subnormals below
  2^-14; IEEE-style infinities and NaNs at exponent 31; largest finite 57344.
* Encoding: round to nearest, ties to even, from the float32 value; results
  beyond the largest finite value saturate to it (never infinity or NaN).
* E4M3 cache: each cached key or value vector gets the float32 scale
  amax / 448 (amax = the largest magnitude of its elements; a zero vector gets
  scale 1), and its codes encode x / scale (float32 division, rounded once), so
  the vector's largest element lands on +-448.  The per-vector scale is the
  granularity the uint8 cache of the quantized oracle uses.
* E5M2 cache: the direct cast of that vLLM option: scale 1, codes encode x.
* Stored like the uint8 cache: codes uint8 [..., d] and float32 pairs
  [..., 2] = (scale, 0) - the zero-point slot of that layout, 0 here - so a
  value reads back as decode(code) * scale.
* The key is quantized after rotation, from its float32 rotated value (the
  rotation sequence of the unquantized oracle, before its storage rounding);
  the value from its input dtype converted to float32.
* Attention is the plain definition of the unquantized oracle, in float64, over
  the dequantized values (each decoded value times its scale is exact in
  float64).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from . import kvc_oracle as O
from . import kvc_quant_oracle as Q

__all__ = ["FORMATS", "fp8_value", "fp8_table", "fp8_encode", "quantize_fp8", "dequantize_fp8",
           "append_contiguous_fp8", "append_paged_fp8", "decode_attention_fp8", "decode_attention_paged_fp8"]

# name -> (exponent bits, mantissa bits, bias, largest finite value, has infinities)
FORMATS = {
    "e4m3": (4, 3, 7, 448.0, False),
    "e5m2": (5, 2, 15, 57344.0, True),
}


def fp8_value(code: int, fmt: str) -> float:
    """The real number (or inf / nan) an 8-bit code stands for, from the format's fields."""
    eb, mb, bias, _, has_inf = FORMATS[fmt]
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    top = (1 << eb) - 1
    if has_inf and e == top:
        return sign * math.inf if m == 0 else math.nan
    if not has_inf and e == top and m == (1 << mb) - 1:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** (1 - bias - mb)
    return sign * (1.0 + m / (1 << mb)) * 2.0 ** (e - bias)


def fp8_table(fmt: str) -> np.ndarray:
    """float64 values of the 256 codes."""
    return np.array([fp8_value(c, fmt) for c in range(256)], dtype=np.float64)


def fp8_encode(x, fmt: str) -> np.ndarray:
    """uint8 codes of float32 values x: nearest representable value, ties to the
    even mantissa, saturating at the largest finite value.  (Inputs are finite.)"""
    eb, mb, bias, vmax, _ = FORMATS[fmt]
    a = np.abs(np.asarray(x, dtype=np.float32).astype(np.float64))
    neg = np.signbit(np.asarray(x, dtype=np.float32))
    emin = 1 - bias                                          # exponent of the smallest normal
    out = np.zeros(a.shape, dtype=np.uint8)
    flat_a, flat_neg, flat_out = a.reshape(-1), neg.reshape(-1), out.reshape(-1)
    for i in range(flat_a.size):
        v = flat_a[i]
        if v == 0.0:
            mag = 0
        else:
            e = max(math.floor(math.log2(v)), emin)
            if 2.0 ** e > v:                                 # (log2 rounding near powers of two)
                e -= 1
            e = max(e, emin)
            ulp = 2.0 ** (e - mb)
            q = v / ulp                                      # exact: v has 24 significant bits at most
            n = math.floor(q)
            r = q - n
            if r > 0.5 or (r == 0.5 and n % 2 == 1):
                n += 1
            if n == (2 << mb):                               # carried into the next binade
                n, e = 1 << mb, e + 1
            value = n * 2.0 ** (e - mb)
            if value > vmax:
                value = vmax
                e = math.floor(math.log2(vmax))
                n = int(vmax / 2.0 ** (e - mb))
            if n < (1 << mb):                                # subnormal (only at e == emin)
                mag = n
            else:
                mag = ((e + bias) << mb) | (n - (1 << mb))
        flat_out[i] = mag | (0x80 if flat_neg[i] else 0)
    return out


def quantize_fp8(x, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """uint8 codes and float32 [..., 2] (scale, 0) pairs of the vectors along the
    last axis of x (float32 arithmetic, each operation rounded once)."""
    v = np.asarray(x, dtype=np.float32)
    if fmt == "e4m3":
        amax = np.max(np.abs(v), axis=-1, keepdims=True)
        scale = (amax / np.float32(FORMATS[fmt][3])).astype(np.float32)
        scale = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
        codes = fp8_encode((v / scale).astype(np.float32), fmt)
    else:
        scale = np.ones(v.shape[:-1] + (1,), np.float32)
        codes = fp8_encode(v, fmt)
    return codes, np.concatenate([scale, np.zeros_like(scale)], axis=-1).astype(np.float32)


def dequantize_fp8(codes, sz, fmt: str) -> np.ndarray:
    """float64 values decode(code) * scale of cached vectors."""
    table = fp8_table(fmt)
    sc = np.asarray(sz, dtype=np.float32)[..., 0:1].astype(np.float64)
    return table[np.asarray(codes, dtype=np.uint8)] * sc


def _quantized_kv(k_new, v_new, p, cos, sin, dtype, style, fmt):
    """Codes and pairs of sequence b's new key (rotated at p) and value, [H_kv, d]."""
    kr = O.rope_rotate_f32(k_new, dtype, cos[p], sin[p], style).astype(np.float32)
    return quantize_fp8(kr, fmt), quantize_fp8(O.to_f32(v_new, dtype), fmt)


def append_contiguous_fp8(k_codes, k_sz, v_codes, v_sz, cached, k_new, v_new, cos, sin, dtype, fmt,
                          style="interleaved", q=None):
    """Quantize rotated k_new and raw v_new into slot cached[b]; q (if given) is
    rotated at the same position as in the unquantized oracle.  Returns new
    arrays; nothing else changes."""
    kc, ks, vc, vs = (np.array(a, copy=True) for a in (k_codes, k_sz, v_codes, v_sz))
    q2 = None if q is None else np.array(q, copy=True)
    for b, p in enumerate(np.asarray(cached).tolist()):
        (ck, sk), (cv, sv) = _quantized_kv(k_new[b], v_new[b], p, cos, sin, dtype, style, fmt)
        kc[b, :, p, :], ks[b, :, p, :] = ck, sk
        vc[b, :, p, :], vs[b, :, p, :] = cv, sv
        if q2 is not None:
            q2[b] = O.rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return kc, ks, vc, vs, q2


def append_paged_fp8(k_codes, k_sz, v_codes, v_sz, block_table, block_size, cached, k_new, v_new,
                     cos, sin, dtype, fmt, style="interleaved", q=None):
    """Paged form: the slot of position p is [table[b][p // bs], :, p % bs]."""
    kc, ks, vc, vs = (np.array(a, copy=True) for a in (k_codes, k_sz, v_codes, v_sz))
    q2 = None if q is None else np.array(q, copy=True)
    for b, p in enumerate(np.asarray(cached).tolist()):
        lb, off = O.paged_location(p, block_size)
        phys = int(block_table[b][lb])
        (ck, sk), (cv, sv) = _quantized_kv(k_new[b], v_new[b], p, cos, sin, dtype, style, fmt)
        kc[phys, :, off, :], ks[phys, :, off, :] = ck, sk
        vc[phys, :, off, :], vs[phys, :, off, :] = cv, sv
        if q2 is not None:
            q2[b] = O.rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return kc, ks, vc, vs, q2


def decode_attention_fp8(q, k_codes, k_sz, v_codes, v_sz, seq_lens, dtype, fmt, scale: Optional[float] = None):
    """Float64 output [B, H_q, d]: the unquantized definition over the
    dequantized first L_b vectors of each group's cache."""
    B = q.shape[0]
    k = np.zeros(k_codes.shape, np.float64)
    v = np.zeros(v_codes.shape, np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        k[b, :, :L] = dequantize_fp8(k_codes[b, :, :L], k_sz[b, :, :L], fmt)
        v[b, :, :L] = dequantize_fp8(v_codes[b, :, :L], v_sz[b, :, :L], fmt)
    return Q._decode_f32_cache(q, k, v, seq_lens, dtype, scale)


def decode_attention_paged_fp8(q, k_codes, k_sz, v_codes, v_sz, block_table, block_size, seq_lens,
                               dtype, fmt, scale: Optional[float] = None):
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
    return decode_attention_fp8(q, kc, ks, vc, vs, seq_lens, dtype, fmt, scale)
