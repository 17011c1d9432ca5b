"""Plain CPU oracle for one decode step of grouped-query attention over a KV cache.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module.  It is written from the pages' definitions,
in float64 wherever the pages leave the precision open, with no tiling, no
splitting and no fusion, so that each function can be read against its source.

Storage dtypes: "f32" arrays are numpy float32; "bf16" arrays are numpy uint16
holding bfloat16 bit patterns (numpy has no bfloat16 type).

Sources (page titles as published; sections as headed on each page):

[GQA]   "Grouped-query attention: berbagi KV head di antara grup query" (nalar.dev):
        section "Jumlah head menentukan batas grup" defines G = H_q / H_kv, the
        group map g(h) = floor(h / G), A_h = softmax(Q_h K_g(h)^T / sqrt(d)) and
        O_h = A_h V_g(h); section "GQA berada di antara MHA dan MQA" gives the end
        cases H_kv = H_q (MHA) and H_kv = 1 (MQA); section "Ukuran KV cache
        mengikuti jumlah KV head" gives 2 * T * H_kv * d stored scalars per layer.
[KVC]   "KV Cache" explainer (lensaml.com): step 3 ("Menyimpan Key dan Value di
        Cache") says the cache is a [batch, kv_heads, tokens, head_dim] tensor
        pair per layer, that a decode step writes one slice along the token axis,
        and that keys are rotated by their position once and stored rotated;
        step 1 and the FAQ say the causal mask makes cached decode equal to full
        recomputation in exact arithmetic; step 5 and the FAQ give the cache bill
        2 * layers * kv_heads * head_dim * bytes * tokens * batch.
[ARCH]  "Arsitektur Inferensi LLM: PagedAttention, KV-Cache & Speculative Decoding"
        (tveniu.com): section 2 (KV bytes per token, GB totals), section 4 (fixed
        blocks of B = 16 tokens mapped through a block table), section 5 (exact
        attention softmax(Q K^T / sqrt(d_k)) V).
[BLOG]  "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략"
        (youngju.dev): the GroupedQueryAttention listing (KV heads broadcast to
        query heads by expand + reshape, i.e. contiguous groups) and the
        PagedKVCache listing (pool [n_blocks, n_heads, block_size, d_k]; logical
        block = pos // block_size, offset = pos % block_size; the last block holds
        len % block_size tokens, or a full block).
[BOOK]  "Solusi Kemacetan Kinerja" (fahmindra.github.io, DeepSeek book, ch. 2):
        section 2.4.2 (the cached decode loop: new q/k/v, load cached K/V,
        concatenate, score, weight V, store K/V back) and listing 2.4 (GQA with
        repeat_interleave and a strict upper-triangular causal mask).

Readings where the pages are silent (each also listed in the design notes):
* RoPE: the pages give neither the pairing nor the frequencies.  Pairs are
  adjacent (2i, 2i+1) ("interleaved") or split halves (i, i + d/2) ("half"); the
  angle of pair i at position p is p * base^(-2i/d); cos/sin come from a float32
  table that the caller supplies.  The rotation is the exact float32 sequence
      r0 = fl(fl(x0 * c) - fl(x1 * s)),   r1 = fl(fl(x0 * s) + fl(x1 * c)),
  with no fused multiply-add, then one round-to-nearest-even into the storage
  dtype.  The query is rotated at the same position with the same table.
* The append slot of sequence b is its cached length c_b (0-based); attention
  then covers L_b = c_b + 1 tokens, the new one included.
* The softmax scale is 1 / sqrt(d), d the per-head dimension.
* Output rounding: the float64 result is rounded once to the storage dtype
  (round to nearest, ties to even).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "DTYPES", "bf16_round_bits", "bf16_to_f32", "to_f32", "to_f64", "round_store",
    "rope_table", "rope_rotate", "rope_rotate_f32", "append_contiguous", "append_paged",
    "decode_attention", "decode_attention_paged", "decode_attention_weights",
    "gather_paged", "causal_attention_full", "kv_elements_per_layer",
    "kv_bytes_per_token", "kv_cache_bytes", "paged_location", "paged_blocks",
    "paged_last_block_fill", "decode_kv_read_bytes", "decode_flops",
]

DTYPES = ("f32", "bf16")

# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact: bf16 is the top half of f32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round_bits(x) -> np.ndarray:
    """Round float64/float32 values to the nearest bfloat16, ties to even.

    Written from the definition of round-to-nearest-even: the candidates are the
    bfloat16 values next to x (found from x's float32 neighbourhood); the one at
    the smaller float64 distance wins, and on a tie the one whose last mantissa
    bit is 0.  NaN maps to a quiet NaN with x's sign.
    """
    x64 = np.asarray(x, dtype=np.float64)
    flat = x64.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    f32 = flat.astype(np.float32)            # within one f32 ulp of x
    u = f32.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    mag = (u & np.uint32(0x7FFF0000)) >> np.uint32(16)   # truncated bf16 magnitude
    best = np.zeros(flat.shape, dtype=np.int64)
    best_d = np.full(flat.shape, np.inf)
    with np.errstate(invalid="ignore"):
        _nearest_bf16(flat, mag, sign, best, best_d)
    out[:] = ((best.astype(np.uint32)) | (sign >> np.uint32(16))).astype(np.uint16)
    nan = np.isnan(flat)
    out[nan] = ((sign[nan] >> np.uint32(16)) | np.uint32(0x7FC0)).astype(np.uint16)
    return out.reshape(x64.shape)


def _nearest_bf16(flat, mag, sign, best, best_d):
    """Update best/best_d in place with the nearest of the three bf16 candidates."""
    for delta in (-1, 0, 1):
        cand = mag.astype(np.int64) + delta
        ok = (cand >= 0) & (cand <= 0x7F80)            # up to +inf magnitude
        c32 = ((np.clip(cand, 0, 0x7F80).astype(np.uint32) << np.uint32(16)) | sign)
        cval = c32.view(np.float32).astype(np.float64)
        dist = np.abs(cval - flat)
        # +inf is "2^128" for distance purposes (RNE overflows past half an ulp)
        inf_c = ok & (np.clip(cand, 0, 0x7F80) == 0x7F80)
        dist = np.where(inf_c, np.abs(np.copysign(2.0 ** 128, flat) - flat), dist)
        dist = np.where(ok, dist, np.inf)
        even = (cand & 1) == 0
        take = (dist < best_d) | ((dist == best_d) & even)
        best[:] = np.where(take, cand, best)
        best_d[:] = np.where(take, dist, best_d)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(a)
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return to_f32(a, dtype).astype(np.float64)


def round_store(x, dtype: str) -> np.ndarray:
    """One rounding (to nearest, ties to even) of float64/float32 values."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return bf16_round_bits(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# RoPE (position rotation applied to keys before they are stored; [KVC] step 3)
# ---------------------------------------------------------------------------


def rope_table(rows: int, d: int, base: float = 10000.0) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin table [rows, d/2]: angle(p, i) = p * base^(-2i/d), float64 -> float32."""
    out_c = np.empty((rows, d // 2), dtype=np.float32)
    out_s = np.empty((rows, d // 2), dtype=np.float32)
    for i in range(d // 2):
        theta = base ** (-(2.0 * i) / d)
        ang = np.arange(rows, dtype=np.float64) * theta
        out_c[:, i] = np.cos(ang)
        out_s[:, i] = np.sin(ang)
    return out_c, out_s


def _pair_index(d: int, style: str):
    half = d // 2
    i = np.arange(half)
    if style == "interleaved":
        return 2 * i, 2 * i + 1
    if style == "half":
        return i, i + half
    raise ValueError(style)


def _fl(x64: np.ndarray) -> np.ndarray:
    """Round an exact float64 result of float32 operands to float32 (one op)."""
    return np.asarray(x64, dtype=np.float64).astype(np.float32).astype(np.float64)


def rope_rotate(x: np.ndarray, dtype: str, cos_row: np.ndarray, sin_row: np.ndarray,
                style: str = "interleaved") -> np.ndarray:
    """Rotate the last axis (head_dim) of stored vectors x by one table row, then
    round once into the storage dtype."""
    return round_store(rope_rotate_f32(x, dtype, cos_row, sin_row, style), dtype)


def rope_rotate_f32(x: np.ndarray, dtype: str, cos_row: np.ndarray, sin_row: np.ndarray,
                    style: str = "interleaved") -> np.ndarray:
    """The rotation before its final rounding: float32 values (held as float64).

    Each op is evaluated in float64 on float32 operands and rounded to float32;
    with 53 >= 2*24 + 2 mantissa bits this is exactly IEEE float32 arithmetic.
    """
    xf = to_f32(x, dtype).astype(np.float64)
    d = xf.shape[-1]
    i0, i1 = _pair_index(d, style)
    c = np.asarray(cos_row, dtype=np.float32).astype(np.float64)
    s = np.asarray(sin_row, dtype=np.float32).astype(np.float64)
    x0, x1 = xf[..., i0], xf[..., i1]
    r0 = _fl(_fl(x0 * c) - _fl(x1 * s))
    r1 = _fl(_fl(x0 * s) + _fl(x1 * c))
    r = np.empty_like(xf)
    r[..., i0] = r0
    r[..., i1] = r1
    return r


# ---------------------------------------------------------------------------
# append: one token slice per sequence ([KVC] step 3; [BOOK] 2.4.2 step 8)
# ---------------------------------------------------------------------------


def append_contiguous(k_cache, v_cache, cached, k_new, v_new, cos, sin, dtype,
                      style="interleaved", q=None):
    """Write rotated k_new and raw v_new at slot cached[b] of [B, H_kv, T, d].

    Returns new arrays (k_cache', v_cache', q') where q' is q rotated at the same
    position (or None).  Nothing else in the caches changes.
    """
    k2, v2 = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    q2 = None if q is None else np.array(q, copy=True)
    for b, p in enumerate(np.asarray(cached).tolist()):
        k2[b, :, p, :] = rope_rotate(k_new[b], dtype, cos[p], sin[p], style)
        v2[b, :, p, :] = v_new[b]
        if q2 is not None:
            q2[b] = rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return k2, v2, q2


def paged_location(pos: int, block_size: int) -> Tuple[int, int]:
    """(logical block, offset in block) of token position pos ([BLOG] PagedKVCache)."""
    return pos // block_size, pos % block_size


def append_paged(k_pool, v_pool, block_table, block_size, cached, k_new, v_new, cos,
                 sin, dtype, style="interleaved", q=None):
    """Paged append: the slot of position p is pool[table[b][p // bs], :, p % bs, :]."""
    k2, v2 = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    q2 = None if q is None else np.array(q, copy=True)
    for b, p in enumerate(np.asarray(cached).tolist()):
        lb, off = paged_location(p, block_size)
        phys = int(block_table[b][lb])
        k2[phys, :, off, :] = rope_rotate(k_new[b], dtype, cos[p], sin[p], style)
        v2[phys, :, off, :] = v_new[b]
        if q2 is not None:
            q2[b] = rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return k2, v2, q2


# ---------------------------------------------------------------------------
# attention for the new token ([GQA] "Jumlah head menentukan batas grup")
# ---------------------------------------------------------------------------


def _head_attention(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(q K^T * scale) V for one query vector; float64 throughout.

    Returns (output [d], weights [L]).  Two passes: the row maximum, then the
    normalised exponentials (the usual safe form of the same softmax).
    """
    if K.shape[0] == 0:
        return np.zeros(qv.shape[-1]), np.zeros(0)
    s = (K @ qv) * scale
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    return (w @ V) / z, w / z


def _check_heads(H_q: int, H_kv: int) -> int:
    if H_kv <= 0 or H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return H_q // H_kv


def decode_attention(q, k_cache, v_cache, seq_lens, dtype, scale: Optional[float] = None):
    """Float64 output [B, H_q, d] of every query head over its group's first L_b tokens.

    q [B, H_q, d] (already rotated), caches [B, H_kv, T, d] in storage dtype.
    Query head h reads KV head floor(h / G).
    """
    B, H_q, d = q.shape
    H_kv = k_cache.shape[1]
    G = _check_heads(H_q, H_kv)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qf = to_f64(q, dtype)
    out = np.zeros((B, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(H_kv):
            K = to_f64(k_cache[b, j, :L], dtype)
            V = to_f64(v_cache[b, j, :L], dtype)
            for h in range(j * G, (j + 1) * G):
                out[b, h], _ = _head_attention(qf[b, h], K, V, sc)
    return out


def decode_attention_weights(q, k_cache, seq_lens, dtype, scale=None):
    """Softmax weights A_h per (b, h) (list of lists of [L_b] float64 arrays)."""
    B, H_q, d = q.shape
    H_kv = k_cache.shape[1]
    G = _check_heads(H_q, H_kv)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qf = to_f64(q, dtype)
    res = []
    for b in range(B):
        L = int(seq_lens[b])
        row = []
        for h in range(H_q):
            K = to_f64(k_cache[b, h // G, :L], dtype)
            _, w = _head_attention(qf[b, h], K, np.zeros((L, d)), sc)
            row.append(w)
        res.append(row)
    return res


def gather_paged(pool, block_table, block_size, b: int, L: int) -> np.ndarray:
    """Logical [H_kv, L, d] view of sequence b, read block by block through the table."""
    nblk = paged_blocks(L, block_size)
    parts = []
    for lb in range(nblk):
        n = block_size if lb < nblk - 1 else paged_last_block_fill(L, block_size)
        parts.append(pool[int(block_table[b][lb]), :, :n, :])
    if not parts:
        return pool[:0].reshape(pool.shape[1], 0, pool.shape[3])
    return np.concatenate(parts, axis=1)


def decode_attention_paged(q, k_pool, v_pool, block_table, block_size, seq_lens, dtype,
                           scale=None):
    """Paged cache: gather each sequence's blocks, then the contiguous definition."""
    B, H_q, d = q.shape
    H_kv = k_pool.shape[1]
    G = _check_heads(H_q, H_kv)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qf = to_f64(q, dtype)
    out = np.zeros((B, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        Kb = gather_paged(k_pool, block_table, block_size, b, L)
        Vb = gather_paged(v_pool, block_table, block_size, b, L)
        for j in range(H_kv):
            K = to_f64(Kb[j], dtype)
            V = to_f64(Vb[j], dtype)
            for h in range(j * G, (j + 1) * G):
                out[b, h], _ = _head_attention(qf[b, h], K, V, sc)
    return out


# ---------------------------------------------------------------------------
# full causal recomputation of a whole sequence (no cache)
# ---------------------------------------------------------------------------


def causal_attention_full(q_raw, k_raw, v, cos, sin, dtype, style="interleaved"):
    """Every position of one sequence at once, with a causal mask.

    q_raw [H_q, n, d], k_raw/v [H_kv, n, d]: raw projections at positions 0..n-1.
    Keys and queries are rotated at their own positions and stored in the storage
    dtype as the append would; scores above the diagonal are masked to -inf (a
    strict upper-triangular mask, as in [BOOK] listing 2.4) before the softmax.
    Returns float64 [H_q, n, d]; row p is what a cached decode step at position p
    must produce.
    """
    H_q, n, d = q_raw.shape
    H_kv = k_raw.shape[0]
    G = _check_heads(H_q, H_kv)
    qr = np.stack([rope_rotate(q_raw[:, t], dtype, cos[t], sin[t], style)
                   for t in range(n)], axis=1)
    kr = np.stack([rope_rotate(k_raw[:, t], dtype, cos[t], sin[t], style)
                   for t in range(n)], axis=1)
    Q, K, V = to_f64(qr, dtype), to_f64(kr, dtype), to_f64(v, dtype)
    mask = np.triu(np.ones((n, n), dtype=bool), k=1)
    out = np.zeros((H_q, n, d))
    for h in range(H_q):
        j = h // G
        S = (Q[h] @ K[j].T) / math.sqrt(d)
        S = np.where(mask, -np.inf, S)
        S = S - S.max(axis=1, keepdims=True)
        W = np.exp(S)
        W = W / W.sum(axis=1, keepdims=True)
        out[h] = W @ V[j]
    return out


# ---------------------------------------------------------------------------
# cache-size and traffic accounting ([GQA] cache size; [ARCH] section 2; [KVC] step 5)
# ---------------------------------------------------------------------------


def kv_elements_per_layer(T: int, H_kv: int, d: int) -> int:
    """Scalars one layer stores for T tokens: keys and values, 2 * T * H_kv * d."""
    return 2 * T * H_kv * d


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, elem_bytes: int) -> int:
    return 2 * n_layers * n_kv_heads * d_head * elem_bytes


def kv_cache_bytes(n_layers, n_kv_heads, d_head, elem_bytes, tokens, batch) -> int:
    return kv_bytes_per_token(n_layers, n_kv_heads, d_head, elem_bytes) * tokens * batch


def paged_blocks(n_tokens: int, block_size: int) -> int:
    return -(-n_tokens // block_size)


def paged_last_block_fill(n_tokens: int, block_size: int) -> int:
    return n_tokens % block_size or block_size


def decode_kv_read_bytes(seq_lens, H_kv: int, d: int, elem_bytes: int) -> int:
    """Bytes of K and V one decode step must read: sum_b L_b * H_kv * d * 2 * e."""
    return int(sum(int(L) for L in seq_lens)) * kv_elements_per_layer(1, H_kv, d) * elem_bytes


def decode_flops(seq_lens, H_q: int, d: int) -> int:
    """Multiply-adds of scores and weighted values, counted as 2 flops each."""
    return 4 * d * H_q * int(sum(int(L) for L in seq_lens))
