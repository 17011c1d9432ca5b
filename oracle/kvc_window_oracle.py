"""Plain CPU oracle for sliding-window decode: the new token attends only the
last W tokens of its sequence.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module.  Like the unquantized oracle it has no
tiling, splitting or fusion; every function can be read against its source.

Source: [BLOG] "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리
효율화 전략" (youngju.dev), the SlidingWindowAttention listing: the new token's
key and value are concatenated to the cache, the cache is cut to its last
window_size tokens when it holds more, and the query attends over what is left
with the plain softmax(q k^T / sqrt(d)) v.  [KVC] "KV Cache" explainer
(lensaml.com), step 6, lists the window among the ways to shrink the cache
(Mistral 7B, 4096 tokens).

Readings (also listed in the design notes):
* W counts the new token: a step whose sequence holds L tokens after the append
  attends tokens [max(0, L - W), L).  W >= L is the unwindowed decode.
* The listing's cut cache is held in one of two layouts:
  - a full cache (contiguous or paged, as the unwindowed oracle's), in which
    the older tokens stay stored and are never read;
  - a ring of T slots (T = W): token t lives in slot t mod T, so the append
    overwrites the token that leaves the window, and the step attends the
    first min(L, T) slots.  They hold the same tokens in another order, which
    attention does not depend on.
* Keys keep the rotation of their own position, applied once at their append
  (the key is stored rotated), so cutting the cache does not re-rotate them.
* The listing has no causal mask for more than one new token; the decode step
  (one query, the last position) needs none.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import kvc_oracle as O

__all__ = ["window_start", "decode_attention_window", "decode_attention_window_paged", "ring_slot",
           "append_ring", "decode_attention_ring"]


def window_start(L: int, window: int) -> int:
    """First attended token of a sequence holding L tokens (the new one
    included) under a window of W tokens (W <= 0: no window)."""
    return max(0, L - window) if window > 0 else 0


def decode_attention_window(q, k_cache, v_cache, seq_lens, window: int, dtype, scale: Optional[float] = None):
    """Float64 [B, H_q, d]: each sequence's query heads over its tokens
    [max(0, L_b - W), L_b) of a full contiguous cache [B, H_kv, T, d]."""
    B, H_q, d = q.shape
    out = np.zeros((B, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        lo = window_start(L, window)
        out[b] = O.decode_attention(q[b:b + 1], k_cache[b:b + 1, :, lo:L], v_cache[b:b + 1, :, lo:L], [L - lo],
                                    dtype, scale)[0]
    return out


def decode_attention_window_paged(q, k_pool, v_pool, block_table, block_size, seq_lens, window: int, dtype,
                                  scale: Optional[float] = None):
    """The same over a paged cache: gather each sequence's tokens through the
    block table, then keep the window."""
    B, H_q, d = q.shape
    out = np.zeros((B, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        lo = window_start(L, window)
        K = O.gather_paged(k_pool, block_table, block_size, b, L)[None, :, lo:L]
        V = O.gather_paged(v_pool, block_table, block_size, b, L)[None, :, lo:L]
        out[b] = O.decode_attention(q[b:b + 1], K, V, [L - lo], dtype, scale)[0]
    return out


def ring_slot(pos: int, T: int) -> int:
    """Slot of token position pos in a ring of T slots."""
    return pos % T


def append_ring(k_ring, v_ring, cached, k_new, v_new, cos, sin, dtype, style="interleaved", q=None):
    """Write rotated k_new and raw v_new of position p = cached[b] into slot
    p mod T of a ring [B, H_kv, T, d]; q (if given) rotated at p.  Returns new
    arrays; nothing else changes."""
    k2, v2 = np.array(k_ring, copy=True), np.array(v_ring, copy=True)
    q2 = None if q is None else np.array(q, copy=True)
    T = k2.shape[2]
    for b, p in enumerate(np.asarray(cached).tolist()):
        s = ring_slot(p, T)
        k2[b, :, s, :] = O.rope_rotate(k_new[b], dtype, cos[p], sin[p], style)
        v2[b, :, s, :] = v_new[b]
        if q2 is not None:
            q2[b] = O.rope_rotate(q[b], dtype, cos[p], sin[p], style)
    return k2, v2, q2


def decode_attention_ring(q, k_ring, v_ring, seq_lens, dtype, scale: Optional[float] = None):
    """Float64 [B, H_q, d] over a ring of T slots: the first min(L_b, T) slots
    (the window of T tokens, in ring order)."""
    T = k_ring.shape[2]
    n = [min(int(L), T) for L in seq_lens]
    return O.decode_attention(q, k_ring, v_ring, n, dtype, scale)
