"""Plain CPU oracle for a decode step with several new tokens per sequence
(speculative verification, chunked prefill): n tokens are appended at once and
each one's query attends causally over the cache and the new tokens up to
itself.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module.  No tiling, splitting or fusion.

Sources:
[ARCH] "Arsitektur Inferensi LLM: PagedAttention, KV-Cache & Speculative
       Decoding" (tveniu.com), section 7: a draft model proposes gamma tokens
       and the target model checks them in one parallel pass (gamma = 5 in its
       worked example, so gamma + 1 = 6 query positions per pass); section 6:
       chunked prefill feeds a prompt in chunks through the same cache.
[KVC]  "KV Cache" explainer (lensaml.com), step 1 and the FAQ: with the causal
       mask, attending from the cache equals recomputing the whole sequence,
       so verifying n tokens at once equals decoding them one at a time.
[BOOK] "Solusi Kemacetan Kinerja" (fahmindra.github.io), listing 2.4: the
       strict upper-triangular causal mask.

Readings (also listed in the design notes):
* Layouts: new keys/values [B, n, H_kv, d], queries and outputs [B, n, H_q, d]
  (token-major, as a model's activations); the cache as the single-token one.
* Token i of sequence b (0 <= i < n) takes position c_b + i: it is stored at
  that slot and rotated (key and query) at that position.
* seq_lens are the lengths after the append (L_b = c_b + n).  Query i attends
  tokens [lo_i, L_b - n + i + 1): the causal mask of [BOOK] listing 2.4 at
  position L_b - n + i, where lo_i = max(0, L_b - n + i + 1 - W) under a
  sliding window of W tokens (0: none), as for a single new token.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import kvc_oracle as O

__all__ = ["query_range", "append_multi", "append_multi_paged", "decode_attention_multi",
           "decode_attention_multi_paged"]


def query_range(L: int, n: int, i: int, window: int = 0):
    """Tokens [lo, hi) query i of n attends in a sequence of L tokens."""
    hi = L - n + i + 1
    lo = max(0, hi - window) if window > 0 else 0
    return lo, hi


def append_multi(k_cache, v_cache, cached, k_new, v_new, cos, sin, dtype, style="interleaved", q=None):
    """Write the n new tokens of each sequence at slots c_b .. c_b + n - 1 of a
    contiguous cache [B, H_kv, T, d]: keys rotated at their positions, values
    as they are; q [B, n, H_q, d] (if given) rotated likewise.  Returns new
    arrays."""
    k2, v2 = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    q2 = None if q is None else np.array(q, copy=True)
    n = k_new.shape[1]
    for b, c in enumerate(np.asarray(cached).tolist()):
        for i in range(n):
            p = c + i
            k2[b, :, p, :] = O.rope_rotate(k_new[b, i], dtype, cos[p], sin[p], style)
            v2[b, :, p, :] = v_new[b, i]
            if q2 is not None:
                q2[b, i] = O.rope_rotate(q[b, i], dtype, cos[p], sin[p], style)
    return k2, v2, q2


def append_multi_paged(k_pool, v_pool, block_table, block_size, cached, k_new, v_new, cos, sin, dtype,
                       style="interleaved", q=None):
    """Paged form: token c_b + i goes to pool[table[b][p // bs], :, p % bs, :]."""
    k2, v2 = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    q2 = None if q is None else np.array(q, copy=True)
    n = k_new.shape[1]
    for b, c in enumerate(np.asarray(cached).tolist()):
        for i in range(n):
            p = c + i
            lb, off = O.paged_location(p, block_size)
            phys = int(block_table[b][lb])
            k2[phys, :, off, :] = O.rope_rotate(k_new[b, i], dtype, cos[p], sin[p], style)
            v2[phys, :, off, :] = v_new[b, i]
            if q2 is not None:
                q2[b, i] = O.rope_rotate(q[b, i], dtype, cos[p], sin[p], style)
    return k2, v2, q2


def decode_attention_multi(q, k_cache, v_cache, seq_lens, dtype, window: int = 0, scale: Optional[float] = None):
    """Float64 [B, n, H_q, d]: query i of sequence b over tokens
    query_range(L_b, n, i, window) of its group's cache."""
    B, n, H_q, d = q.shape
    out = np.zeros((B, n, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(n):
            lo, hi = query_range(L, n, i, window)
            out[b, i] = O.decode_attention(q[b:b + 1, i], k_cache[b:b + 1, :, lo:hi], v_cache[b:b + 1, :, lo:hi],
                                           [hi - lo], dtype, scale)[0]
    return out


def decode_attention_multi_paged(q, k_pool, v_pool, block_table, block_size, seq_lens, dtype, window: int = 0,
                                 scale: Optional[float] = None):
    """Paged cache: gather each sequence's tokens, then the contiguous form."""
    B, n, H_q, d = q.shape
    out = np.zeros((B, n, H_q, d))
    for b in range(B):
        L = int(seq_lens[b])
        K = O.gather_paged(k_pool, block_table, block_size, b, L)[None]
        V = O.gather_paged(v_pool, block_table, block_size, b, L)[None]
        out[b] = decode_attention_multi(q[b:b + 1], K, V, [L], dtype, window, scale)[0]
    return out
