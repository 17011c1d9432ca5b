"""Plain CPU oracle for a decode step of multi-head latent attention (MLA) over
a latent cache.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module.  It computes the listing's arithmetic as
written: the whole cache is up-projected to per-head keys and values, then the
plain attention definition runs per head.  No absorption, tiling or splitting.

Source: [BLOG] "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리
효율화 전략" (youngju.dev), the MultiHeadLatentAttention listing:
* the cache holds, per token, a latent c_kv (d_latent values, the down-
  projection of the token) and k_rope (rope_dim values), concatenated to the
  cache along the token axis each step; its size is B * S * (d_latent +
  rope_dim) elements, d_latent / (2 * n_heads * d_k) of a full per-head cache
  (the listing's comment, rope part aside);
* keys and values are recovered per head by the up-projections W_uk, W_uv
  (nn.Linear(d_latent, n_heads * d_k), with bias), viewed as [S, n_heads, d_k];
* attention is softmax(q k^T / sqrt(d_k)) v per head, d_k = d_model / n_heads.

Readings (also listed in the design notes):
* The listing computes k_rope and stores it in the cache but never uses it in
  the attention (the page is inconsistent here).  The attention follows the
  listing as written: k_rope is stored by the append and not read.
* Neither c_kv nor k_rope is rotated anywhere in the listing; the append
  stores both as given.
* Cache layout: one array [B, T, d_latent + rope_dim] per layer, each token's
  row holding c_kv then k_rope (the listing's (c_kv, k_rope) pair, packed).
* The new token's latent is appended before attention (the listing
  concatenates, then attends), so a step attends over L = c + 1 tokens.
* Weights follow nn.Linear: W [out, in] with bias [out]; y = W x + b.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import kvc_oracle as O

__all__ = ["append_mla", "up_project", "decode_attention_mla", "decode_attention_mla_heads",
           "mla_cache_bytes_per_token"]


def append_mla(cache, cached, c_kv_new, k_rope_new):
    """Store token c_b's latent row [c_kv | k_rope] at slot c_b of each
    sequence's cache [B, T, d_latent + rope_dim].  Returns a new array."""
    c2 = np.array(cache, copy=True)
    dl = c_kv_new.shape[-1]
    for b, p in enumerate(np.asarray(cached).tolist()):
        c2[b, p, :dl] = c_kv_new[b]
        c2[b, p, dl:] = k_rope_new[b]
    return c2


def up_project(c_kv, W, bias, n_heads: int, d_k: int):
    """Per-head vectors from latents, as the listing's W(c).view(S, n_heads, d_k):
    float64 [n_heads, S, d_k] from c_kv [S, d_latent] (float64)."""
    y = c_kv @ W.T + bias                      # [S, n_heads * d_k]
    return y.reshape(c_kv.shape[0], n_heads, d_k).transpose(1, 0, 2)


def decode_attention_mla(q, cache, seq_lens, W_uk, b_uk, W_uv, b_uv, d_latent: int, dtype,
                         scale: Optional[float] = None):
    """Float64 [B, n_heads, d_k]: head h of sequence b over its first L_b
    tokens, with keys / values up-projected from the cached latents.

    q [B, n_heads, d_k] and cache in storage dtype; W_uk, W_uv [n_heads * d_k,
    d_latent] and biases [n_heads * d_k] in storage dtype.
    """
    B, H, d_k = q.shape
    sc = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    qf = O.to_f64(q, dtype)
    Wk, bk = O.to_f64(W_uk, dtype), O.to_f64(b_uk, dtype)
    Wv, bv = O.to_f64(W_uv, dtype), O.to_f64(b_uv, dtype)
    out = np.zeros((B, H, d_k))
    for b in range(B):
        L = int(seq_lens[b])
        c = O.to_f64(cache[b, :L, :d_latent], dtype)
        K = up_project(c, Wk, bk, H, d_k)
        V = up_project(c, Wv, bv, H, d_k)
        for h in range(H):
            out[b, h], _ = O._head_attention(qf[b, h], K[h], V[h], sc)
    return out


def decode_attention_mla_heads(q, cache, seq_lens, W_uk, b_uk, W_uv, b_uv, d_latent: int, dtype, pairs,
                               scale: Optional[float] = None):
    """Float64 [len(pairs), d_k]: decode_attention_mla's output at the listed
    (b, h) pairs only.  Head h's keys and values come from its own d_k rows
    of W_uk and W_uv (the rows the listing's view(S, n_heads, d_k) gives it),
    so a long cache is up-projected for the sampled heads alone."""
    d_k = q.shape[2]
    sc = (1.0 / math.sqrt(d_k)) if scale is None else float(scale)
    out = np.zeros((len(pairs), d_k))
    cached = {}
    for n, (b, h) in enumerate(pairs):
        L = int(seq_lens[b])
        if b not in cached:
            cached[b] = O.to_f64(cache[b, 0:L, 0:d_latent], dtype)
        rows = slice(h * d_k, (h + 1) * d_k)
        K = up_project(cached[b], O.to_f64(W_uk[rows], dtype), O.to_f64(b_uk[rows], dtype), 1, d_k)[0]
        V = up_project(cached[b], O.to_f64(W_uv[rows], dtype), O.to_f64(b_uv[rows], dtype), 1, d_k)[0]
        out[n], _ = O._head_attention(O.to_f64(q[b, h], dtype), K, V, sc)
    return out


def mla_cache_bytes_per_token(d_latent: int, rope_dim: int, elem_bytes: int) -> int:
    """Bytes one token adds to one layer's latent cache: (d_latent + rope_dim) * e."""
    return (d_latent + rope_dim) * elem_bytes
