"""MI355X-native decode step of grouped-query attention over a KV cache.

The work runs in libkvc.so (hand-written HIP for gfx950 behind the C ABI in
include/kvc.h); this package only marshals torch tensors into it:

    append(k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin, q=..., block_table=...)
    decode_attn(q, k_cache, v_cache, seq_lens, max_seq_len)
    decode_attn_paged(q, k_pool, v_pool, block_table, seq_lens, max_seq_len)
    decode_step(q, k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin, max_seq_len, ...)
    step = prepare_decode_step(...same arguments...); step()   # checked once, launched per call

with a sliding window (the last `window` tokens of a full cache, or a ring of slots):

    append_ring(k_ring, v_ring, positions, k_new, v_new, rope_cos, rope_sin, q=...)
    decode_attn_window(q, k_cache, v_cache, seq_lens, max_seq_len, window, ring=..., block_table=...)
    decode_step_window(q, k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin, max_seq_len, window, ...)

several new tokens per sequence (speculative verification, chunked prefill):

    append_multi(k_cache, v_cache, positions, k_new, v_new, rope_cos, rope_sin, q=..., block_table=...)
    decode_attn_multi(q, k_cache, v_cache, seq_lens, max_seq_len, window=..., block_table=...)

and, for a uint8 quantized cache (codes plus a (step, zero point) pair per vector):

    append_u8(k_codes, k_sz, v_codes, v_sz, positions, k_new, v_new, rope_cos, rope_sin, ...)
    decode_attn_u8(q, k_codes, k_sz, v_codes, v_sz, seq_lens, max_seq_len)
    decode_attn_paged_u8(q, k_codes, k_sz, v_codes, v_sz, block_table, seq_lens, max_seq_len)
    decode_step_u8(q, k_codes, k_sz, v_codes, v_sz, positions, k_new, v_new, rope_cos, rope_sin, max_seq_len, ...)

and for a latent cache (multi-head latent attention, one [c_kv | k_rope] row per token):

    append_mla(cache, positions, c_kv_new, k_rope_new)
    decode_attn_mla(q, cache, seq_lens, max_seq_len, w_uk, w_uv, b_uv)
    decode_step_mla(q, cache, positions, c_kv_new, k_rope_new, max_seq_len, w_uk, w_uv, b_uv)
"""
from .api import (KVC_BF16, KVC_F32, KVC_U8, KvcError, PreparedCall, append, append_multi,  # noqa: F401
                  append_ring, append_u8, balanced, compact, decode_attn, decode_attn_multi, decode_attn_paged,
                  decode_attn_paged_u8, decode_attn_u8, FP8_FORMATS, append_fp8, decode_attn_fp8,
                  decode_attn_paged_fp8, decode_step_fp8, prepare_decode_step_fp8, decode_attn_window, decode_step, decode_step_noalloc, decode_step_u8,
                  decode_step_window, merge_launch, multi_split_tokens, multi_workspace_bytes, noalloc_max_bytes,
                  prepare_decode_step, prepare_decode_step_u8, profile_next_decode, split_tokens, window_span,
                  workspace_bytes, workspace_zeroed_bytes)
from .api import (append_mla, decode_attn_mla, decode_step_mla, mla_split_tokens,  # noqa: F401
                  mla_workspace_bytes)
from ._lib import LIB_PATH, load  # noqa: F401
