/*
 * kvc.h - C ABI of libkvc: one autoregressive decode step of grouped-query
 * attention over a KV cache, on an AMD Instinct MI355X (gfx950).
 *
 * A decode step is two operations on one stream:
 *   1. kvc_append: rotate the new token's key (RoPE) and store it, with the
 *      token's value, as one slice along the token axis of the cache; the same
 *      call can rotate the token's query in place.
 *   2. kvc_decode_attn / kvc_decode_attn_paged: every query head h attends over
 *      the cached keys/values of its group g(h) = floor(h / G), G = H_q / H_kv:
 *      O_h = softmax(q_h K_g(h)^T * scale) V_g(h).
 * kvc_decode_step does both in one call (and, for the common shapes, in one
 * streaming kernel).
 *
 * Definitions followed (page titles as published):
 *  - "Grouped-query attention: berbagi KV head di antara grup query" (nalar.dev),
 *    section "Jumlah head menentukan batas grup": G, g(h), A_h and O_h; section
 *    "GQA berada di antara MHA dan MQA": H_kv = H_q is MHA, H_kv = 1 is MQA.
 *  - "KV Cache" explainer (lensaml.com), step 3: the cache is a pair of
 *    [batch, kv_heads, tokens, head_dim] tensors per layer, each decode step
 *    writes one slice along the token axis, and keys are rotated by position
 *    once and stored rotated.
 *  - "Arsitektur Inferensi LLM: PagedAttention, KV-Cache & Speculative
 *    Decoding" (tveniu.com), section 4: the cache split into fixed blocks of
 *    tokens placed anywhere in memory and found through a per-sequence table.
 *  - "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략"
 *    (youngju.dev), PagedKVCache listing: pool [n_blocks, n_heads, block_size,
 *    head_dim], logical block pos / block_size, offset pos % block_size; and
 *    its QuantizedKVCache listing (the *_u8 entry points): uint8 codes with a
 *    per-vector step and zero point; its SlidingWindowAttention listing (the
 *    *_window and *_ring entry points): attention over the last W tokens.
 *  - "Arsitektur Inferensi LLM: PagedAttention, KV-Cache & Speculative
 *    Decoding" (tveniu.com), sections 6 and 7 (the *_multi entry points):
 *    several new tokens per sequence in one pass - the target model checking
 *    gamma drafted tokens, or a prompt chunk - each attending causally.
 *  - "KV Cache 최적화 심층 분석" (youngju.dev), MultiHeadLatentAttention listing
 *    (the *_mla entry points): a latent cache of one [c_kv | k_rope] row per
 *    token, keys and values recovered per head by the up-projections W_uk,
 *    W_uv.
 *
 * Conventions for every entry point:
 *  - All tensors are dense, row-major, in DEVICE memory, owned by the caller.
 *    The library allocates nothing and keeps no per-call state.
 *  - dtype: KVC_BF16 (bfloat16 q/K/V/out, float32 accumulation) or KVC_F32.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *    and never synchronise.  Sizes are checked on the host before anything is
 *    launched: a non-OK status means nothing was enqueued, and kvc_last_error()
 *    (thread-local) says why.  Values that live in device memory (positions,
 *    lengths, block ids) cannot be checked on the host; the kernels clamp them
 *    so that every access stays inside the buffers described by the sizes
 *    passed in, but the results for out-of-contract values are unspecified.
 *  - Output buffers must not alias inputs.  Concurrent calls are safe when
 *    they do not share output or workspace buffers.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 14

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_NULL = 1,        /* a required pointer is NULL                       */
    KVC_ERR_SHAPE = 2,       /* inconsistent sizes (H_q % H_kv, capacity, ...)   */
    KVC_ERR_UNSUPPORTED = 3, /* valid request this build does not implement      */
    KVC_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned       */
    KVC_ERR_HIP = 5          /* a HIP runtime call failed                        */
} kvc_status;

/* KVC_U8 names the quantized cache of kvc_append_u8 / kvc_decode_attn*_u8
 * (uint8 codes, bf16 queries and outputs), KVC_FP8_E4M3 / KVC_FP8_E5M2 the FP8
 * caches of the *_fp8 calls; the sizing and plan queries
 * (kvc_decode_workspace_bytes, kvc_decode_split_tokens, ...) take them as a
 * dtype, and the *_fp8 calls as their format argument. */
typedef enum kvc_dtype {
    KVC_F32 = 0,
    KVC_BF16 = 1,
    KVC_U8 = 2,
    KVC_FP8_E4M3 = 3,
    KVC_FP8_E5M2 = 4
} kvc_dtype;

/* How RoPE pairs the head dimension: (2i, 2i+1), or (i, i + d/2). */
typedef enum kvc_rope_style { KVC_ROPE_INTERLEAVED = 0, KVC_ROPE_HALF = 1 } kvc_rope_style;

/* KVC_ABI_VERSION of the loaded library. */
int kvc_abi_version(void);

/* Static text for a status code (never NULL). */
const char* kvc_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* kvc_last_error(void);

/*
 * Timing aid.  The next kvc_decode_attn / kvc_decode_attn_paged call made on
 * this thread launches its streaming (split) kernel with start_event and
 * stop_event attached (hipExtLaunchKernel), so the two events bracket exactly
 * that kernel and hipEventElapsedTime gives its duration.  Both are hipEvent_t
 * handles owned by the caller (or NULL).  One-shot: the next decode call, even
 * a failing one, clears them.
 */
void kvc_profile_next_decode(void* start_event, void* stop_event);

/*
 * Measurement aid: a plain streaming read of `bytes` (a multiple of 16) from
 * device buffer `buf` by `workgroups` workgroups of 256 threads, each reading
 * one contiguous slice with 16-byte loads, with the default cache policy or,
 * when `nontemporal` is nonzero, the non-temporal one (the policy of the
 * decode kernels' K/V loads).  Its rate is the practical HBM read ceiling
 * that a read-bound kernel such as decode attention can approach.  `sink` is
 * a device buffer of `workgroups` uint32 (written almost never).
 */
kvc_status kvc_hbm_read_probe(const void* buf, size_t bytes, void* sink, int workgroups, int nontemporal,
                              void* stream);

/*
 * kvc_append - write the new token of every sequence into the cache.
 *
 * For sequence b, p = positions[b] is the slot (the number of tokens cached
 * before this step).  For every KV head j and pair i of the head dimension,
 * with x0, x1 the pair of k_new[b, j, :] (style picks the pair), c =
 * rope_cos[p, i], s = rope_sin[p, i], the stored key is
 *     r0 = (x0*c) - (x1*s),   r1 = (x0*s) + (x1*c)
 * evaluated in float32 one rounded operation at a time (no fused multiply-add)
 * and rounded to nearest-even into the storage dtype.  v_new[b, j, :] is copied
 * bit for bit.  If q_inout is not NULL, q_inout[b, h, :] is rotated in place in
 * the same way at the same position.  No other cache element changes.
 *
 * Cache layout:
 *   block_table == NULL: contiguous k_cache/v_cache [B, H_kv, T_max, d];
 *                        the slot is [b, j, p, :].  Requires p < T_max.
 *   block_table != NULL: pools k_cache/v_cache [num_blocks, H_kv, block_size, d]
 *                        and int32 block_table [B, max_blocks_per_seq]; the slot
 *                        is [block_table[b][p / block_size], j, p % block_size, :].
 *                        Requires p < max_blocks_per_seq * block_size and that
 *                        table entry in [0, num_blocks).  T_max is ignored.
 * Positions outside [0, min(capacity, rope_rows)), or a block id outside
 * [0, num_blocks), make the kernel skip that sequence's writes.
 *
 * Arguments: positions int32 [B]; k_new, v_new [B, H_kv, d]; q_inout [B, H_q, d]
 * or NULL; rope_cos, rope_sin float32 [rope_rows, d/2] (row p holds the
 * cos/sin of the pair angles at position p).  d must be even.
 */
kvc_status kvc_append(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                      void* k_cache, void* v_cache, int T_max,
                      const int32_t* block_table, int block_size, int max_blocks_per_seq,
                      int num_blocks, const int32_t* positions,
                      const void* k_new, const void* v_new, void* q_inout,
                      const float* rope_cos, const float* rope_sin, int rope_rows,
                      int rope_style, void* stream);

/*
 * Bytes of workspace kvc_decode_attn / kvc_decode_attn_paged / kvc_decode_step
 * need for these sizes and this split_tokens (0 = the library's choice).  May
 * be 0.  Returns (size_t)-1 for invalid sizes (kvc_last_error says why).
 *
 * pool_tokens is num_blocks * block_size for a paged cache (the pool's token
 * capacity, which the library's split choice takes into account) and 0 for a
 * contiguous cache; pass the same sizes as the decode call.
 *
 * The workspace holds the per-split partial results (running max and sum
 * per query head, weighted value sums; under the balanced schedule, two
 * partial rows per query head of a group for each of its workgroups) and, in
 * its first
 * kvc_workspace_zeroed_bytes() bytes, one arrival counter per (sequence, KV
 * head) that the splits of the bf16 matrix-core kernel count themselves in
 * with: the last split of each to finish merges the partials, in the same
 * launch.  Those first bytes must be zero before a workspace is first used
 * (e.g. hipMemset once after allocating it); every call that runs to
 * completion leaves them zero again, so a workspace needs no clearing between
 * calls.  The rest needs no initialisation and means nothing between calls.
 * Calls that overlap in time must not share a workspace.
 */
size_t kvc_decode_workspace_bytes(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                                  int max_seq_len, long long pool_tokens, int split_tokens);

/*
 * Length of the prefix of every decode and latent-cache workspace that holds
 * the split kernels' arrival counters (64 KiB): zero before the workspace's
 * first use, and left zero by every completed call.  A workspace of 0 bytes
 * (kvc_decode_workspace_bytes returned 0) has none.
 */
size_t kvc_workspace_zeroed_bytes(void);

/*
 * The split length (tokens per workgroup) a decode call with these sizes
 * uses: split_tokens itself when it is positive, else the library's choice.
 * Arguments as for kvc_decode_workspace_bytes; returns -1 for invalid sizes.
 *
 * The library's choice: one round of workgroups that occupies every compute
 * unit equally (as many workgroups as the device holds at once for this
 * kernel, spread over B * H_kv sequence-head pairs); for a paged pool much
 * smaller than B * max_seq_len (ragged lengths), about four rounds of
 * shorter splits; never fewer than 32 * (H_q / H_kv) tokens, so that the
 * partial results stay a few percent of the bytes read.  With the library's
 * choice over a contiguous bf16 cache, the last split of a sequence also
 * takes a remainder shorter than one loop step of the kernel (64 tokens up
 * to head_dim 128, else 128): 8193 tokens in splits of 4096 are two splits,
 * of 4096 and 4097 tokens.  Under the compacted schedule (kvc_decode_compact)
 * this is the shortest split length the kernel may pick.
 */
int kvc_decode_split_tokens(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                            long long pool_tokens, int split_tokens);

/*
 * Whether a decode call with these sizes (arguments as for
 * kvc_decode_workspace_bytes) launches a separate merge kernel after the
 * streaming kernel: 1 if it does, 0 if not (one split per sequence, or a plan
 * whose workgroups all fit in one round, where the last split of each
 * (sequence, KV head) merges in the streaming kernel itself; the bf16 and
 * uint8 matrix-core kernels only, and always under the balanced schedule);
 * -1 for invalid sizes.
 */
int kvc_decode_merge_launch(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                            long long pool_tokens, int split_tokens);

/*
 * Whether a single-token decode with these sizes (arguments as for
 * kvc_decode_workspace_bytes; a call without a window) runs the balanced
 * schedule: 1 if it does, 0 if it uses splits of the planned length, -1 for
 * invalid sizes.
 *
 * The balanced schedule (bf16, head_dim 64 or 128, at most 512 sequences,
 * the library's split choice, paged pools of blocks of a multiple of 16
 * tokens): every workgroup reads the B lengths, lays the loop steps of all
 * (sequence, KV head) units out in one list and streams an equal share of it,
 * so ragged lengths cost no idle or short workgroups (the units are the
 * partition of "Grouped-query attention: berbagi KV head di antara grup
 * query", nalar.dev, section "Jumlah head menentukan batas grup"; their
 * partial results merge by log-sum-exp as the splits' do).  The library uses
 * it for paged pools much smaller than B * max_seq_len (ragged lengths); a
 * call with a sliding window, several new tokens or another block size takes
 * the split plan, whose workspace the returned size also covers.
 */
int kvc_decode_balanced(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                        long long pool_tokens, int split_tokens);

/*
 * Whether a single-token decode with these sizes (arguments as for
 * kvc_decode_workspace_bytes) runs the compacted schedule: 1 if it does, 0 if
 * not, -1 for invalid sizes.
 *
 * The compacted schedule (bf16 matrix-core kernel, contiguous cache, at most
 * 256 sequences, B * H_kv at most half the workgroups the device holds at
 * once, the library's split choice) replaces split plans that would take
 * several rounds of workgroups.  The host knows only max_seq_len, so such a
 * plan, sized for the longest sequence, leaves many splits past the end of
 * shorter ones.  Instead every workgroup reads the B lengths and picks the
 * split length itself: the shortest multiple of the kernel's loop step, at
 * least kvc_decode_split_tokens, whose splits of all (sequence, KV head)
 * units fit in one round of workgroups; the splits that exist take the first
 * workgroup indices, and the merge kernel, which derives the same length from
 * the same lengths, combines them (the split and merge of "Arsitektur
 * Inferensi LLM", tveniu.com, section 5, with the units of "Grouped-query
 * attention: berbagi KV head di antara grup query", nalar.dev, section
 * "Jumlah head menentukan batas grup").  The workspace is that of the
 * shortest split length.
 */
int kvc_decode_compact(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                       long long pool_tokens, int split_tokens);

/*
 * kvc_decode_attn - attention of the new token over a contiguous cache.
 *
 * out[b, h, :] = sum_t w_t V[b, g(h), t, :] over t < L_b = seq_lens[b], with
 * w = softmax_t(scale * <q[b, h, :], K[b, g(h), t, :]>), g(h) = h / (H_q / H_kv).
 * q is the (already rotated) query [B, H_q, d]; k_cache, v_cache [B, H_kv,
 * T_max, d]; seq_lens int32 [B] with 0 <= L_b <= max_seq_len <= T_max (L_b = 0
 * gives zeros); scale <= 0 means 1/sqrt(d); out [B, H_q, d] in dtype.
 * Slots at or past L_b are never read.
 *
 * The token axis is cut into splits of split_tokens tokens (0 = library
 * heuristic); each split is one workgroup per (sequence, KV head) and, when a
 * sequence has more than one split, a second kernel on the same stream merges
 * them exactly by their log-sum-exp.  The result does not depend on the split
 * count beyond float32 rounding.
 */
kvc_status kvc_decode_attn(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                           const void* q, const void* k_cache, const void* v_cache, int T_max,
                           const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                           int split_tokens, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * kvc_decode_attn_paged - the same attention over a paged cache.
 *
 * k_pool, v_pool [num_blocks, H_kv, block_size, d]; block_table int32
 * [B, max_blocks_per_seq]: token t of sequence b lives in block
 * block_table[b][t / block_size] at offset t % block_size.  Entries past
 * ceil(L_b / block_size) are never read.  Requires max_seq_len <=
 * max_blocks_per_seq * block_size.  Blocks may be shared between sequences.
 */
kvc_status kvc_decode_attn_paged(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 int num_blocks, int block_size, const int32_t* block_table,
                                 int max_blocks_per_seq, const int32_t* seq_lens,
                                 int max_seq_len, float scale, void* out, int split_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_step - one whole decode step: kvc_append followed by the
 * attention of the new token, as one call.
 *
 * Same result as kvc_append(..., q_inout = copy of q ...) followed by
 * kvc_decode_attn[_paged] with seq_lens[b] = positions[b] + 1, bit for bit:
 * the new token's key is rotated and stored with its value at slot
 * positions[b], the query is rotated at the same position (written to
 * q_rot_out), and every query head attends over the positions[b] + 1 cached
 * tokens, the new one included.  For bf16 with head_dim 64/128/256 and
 * G <= 32 the append runs inside the streaming attention kernel (q is
 * rotated in registers; the workgroup whose split holds the new token uses
 * the rotated key and the value from registers for that token and stores
 * them to the cache after its pass).  Over a contiguous cache the vector
 * kernel of the other shapes does the same (queries and the new key rotated
 * in LDS).  A paged cache without the matrix-core kernel, and a ring, run
 * the append kernel first.
 *
 * q is the raw query [B, H_q, d] (not modified); q_rot_out [B, H_q, d]
 * (required) receives the rotated query.  Cache arguments as in kvc_append
 * (block_table == NULL: contiguous [B, H_kv, T_max, d]; else paged pools).
 * max_seq_len must be >= every positions[b] + 1; a position outside the cache
 * or the rotation table writes nothing and gives zeros for that sequence.
 * Workspace as for kvc_decode_attn (kvc_decode_workspace_bytes with the same
 * sizes, max_seq_len and pool_tokens).
 */
kvc_status kvc_decode_step(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                           const void* q, void* q_rot_out, void* k_cache, void* v_cache, int T_max,
                           const int32_t* block_table, int block_size, int max_blocks_per_seq,
                           int num_blocks, const int32_t* positions, const void* k_new,
                           const void* v_new, const float* rope_cos, const float* rope_sin,
                           int rope_rows, int rope_style, int max_seq_len, float scale, void* out,
                           int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_step_noalloc - kvc_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * Arguments, results and errors as kvc_decode_step, without the workspace:
 * the split partials go to a fixed array of device memory inside the library
 * (kvc_decode_step_noalloc_max_bytes() bytes, 32 MiB; one copy per device,
 * held until the process ends).  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); the caller passes every input and
 * output.  The first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress, the device current).
 *
 * Limit: a call whose partials would need more than the array holds (as
 * kvc_decode_workspace_bytes reports for the same sizes) returns
 * KVC_ERR_WORKSPACE before anything is launched; a longer split_tokens, or
 * kvc_decode_step with a workspace of the caller's, serves such sizes.
 *
 * Every call on one device shares that device's array, which keeps whatever
 * the last call left in it.  Its first kvc_workspace_zeroed_bytes() bytes are
 * the arrival counters of a workspace (zero when the library is loaded, and
 * left zero by every completed call); the rest needs no clearing, since every
 * call writes the partials it reads.  Calls that overlap in time on one device - on
 * different streams, or from different threads - race on it and give
 * unspecified results; serialise them (one stream, or events).
 */
kvc_status kvc_decode_step_noalloc(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                                   const void* q, void* q_rot_out, void* k_cache, void* v_cache, int T_max,
                                   const int32_t* block_table, int block_size, int max_blocks_per_seq,
                                   int num_blocks, const int32_t* positions, const void* k_new,
                                   const void* v_new, const float* rope_cos, const float* rope_sin,
                                   int rope_rows, int rope_style, int max_seq_len, float scale, void* out,
                                   int split_tokens, void* stream);

/* Bytes of split partials kvc_decode_step_noalloc can hold (its fixed array). */
size_t kvc_decode_step_noalloc_max_bytes(void);

/*
 * Sliding window: the new token attends only the last `window` tokens of its
 * sequence, itself included - the SlidingWindowAttention listing of "KV Cache
 * 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략"
 * (youngju.dev), which concatenates the new key and value and cuts the cache
 * to its last window_size tokens.  That cut cache is held either as
 *   - a full cache (contiguous, or paged through a block table, laid out as
 *     for kvc_decode_attn[_paged]): a sequence holding L tokens attends tokens
 *     [max(0, L - window), L); the older ones stay stored and are never read
 *     (window 0: no window); or
 *   - a ring (contiguous only, ring = 1): k/v [B, H_kv, T_max, d], token t in
 *     slot t % T_max, written by kvc_append_ring; the window is T_max (pass
 *     window 0 or T_max) and the slots [0, min(L, T_max)) are attended.
 *     Attention does not depend on the order of the tokens, so this equals
 *     the window over a full cache.
 */

/*
 * kvc_append_ring - kvc_append into a contiguous ring of T_max slots: the new
 * token of position p = positions[b] goes to slot p % T_max (replacing the
 * token p - T_max, which has left the window); its key and q_inout (if not
 * NULL) are rotated at position p itself.  Positions must be in [0,
 * rope_rows) (others write nothing); they may exceed T_max.
 */
kvc_status kvc_append_ring(kvc_dtype dtype, int B, int H_q, int H_kv, int d, void* k_ring, void* v_ring,
                           int T_max, const int32_t* positions, const void* k_new, const void* v_new,
                           void* q_inout, const float* rope_cos, const float* rope_sin, int rope_rows,
                           int rope_style, void* stream);

/*
 * The token span the splits of a windowed call cover: min(max_seq_len,
 * T_max) for a ring, min(max_seq_len, window + 15) for a window over a full
 * cache (the paged kernels start their splits at a multiple of 16 tokens),
 * max_seq_len without either.  Pass it as max_seq_len to
 * kvc_decode_workspace_bytes / kvc_decode_split_tokens when sizing the
 * workspace of kvc_decode_attn_window / kvc_decode_step_window.  -1 for
 * invalid sizes.
 */
int kvc_window_span(int max_seq_len, int window, int ring, int T_max);

/*
 * kvc_decode_attn_window - kvc_decode_attn (block_table == NULL) or
 * kvc_decode_attn_paged over the window described above.  Arguments as for
 * those calls, plus window (>= 0) and ring (0 or 1; contiguous only; then
 * max_seq_len may exceed T_max).  seq_lens are the sequences' full lengths L
 * (tokens ever appended, the new one included).
 */
kvc_status kvc_decode_attn_window(kvc_dtype dtype, int B, int H_q, int H_kv, int d, const void* q,
                                  const void* k_cache, const void* v_cache, int T_max, const int32_t* block_table,
                                  int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* seq_lens,
                                  int max_seq_len, int window, int ring, float scale, void* out, int split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_step_window - kvc_decode_step with a window: the same append
 * (kvc_append_ring's slot when ring = 1) and the attention of the new token
 * over its window, with L = positions[b] + 1.  Bit for bit the result of the
 * append followed by kvc_decode_attn_window.  For bf16 with head_dim
 * 64/128/256 and G <= 32 over a full cache the append runs inside the
 * streaming kernel; a ring runs the append kernel first.
 */
kvc_status kvc_decode_step_window(kvc_dtype dtype, int B, int H_q, int H_kv, int d, const void* q, void* q_rot_out,
                                  void* k_cache, void* v_cache, int T_max, const int32_t* block_table,
                                  int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* positions,
                                  const void* k_new, const void* v_new, const float* rope_cos,
                                  const float* rope_sin, int rope_rows, int rope_style, int max_seq_len,
                                  int window, int ring, float scale, void* out, int split_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Several new tokens per sequence (speculative verification of drafted
 * tokens, chunked prefill): token i (0 <= i < n) of sequence b takes position
 * positions[b] + i; its query attends the cache and the new tokens up to
 * itself (causal), i.e. tokens [lo_i, L_b - n + i + 1) with L_b = seq_lens[b]
 * (the length after the append, so L_b >= n) and lo_i = max(0, L_b - n + i +
 * 1 - window) (window 0: lo_i = 0).  Layouts are token-major:
 * k_new, v_new [B, n, H_kv, d]; q, q_inout, out [B, n, H_q, d].  n = 1 is the
 * single-token step.  Decode: bf16 only, head_dim 64, 128 or 256; the G * n
 * query rows of a KV group are served 32 at a time from one pass over its
 * cache (ceil(G * n / 32) passes).
 */

/*
 * kvc_append_multi - kvc_append for n tokens per sequence: token i goes to
 * slot positions[b] + i (contiguous, or through the block table), its key
 * and q_inout[b, i] (if not NULL) rotated at that position.  Tokens whose
 * position is outside the cache or the table write nothing.
 */
kvc_status kvc_append_multi(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, void* k_cache, void* v_cache,
                            int T_max, const int32_t* block_table, int block_size, int max_blocks_per_seq,
                            int num_blocks, const int32_t* positions, const void* k_new, const void* v_new,
                            void* q_inout, const float* rope_cos, const float* rope_sin, int rope_rows,
                            int rope_style, void* stream);

/*
 * Workspace bytes and split length of kvc_decode_attn_multi with these sizes
 * (as kvc_decode_workspace_bytes / kvc_decode_split_tokens; pool_tokens as
 * there).  (size_t)-1 / -1 for invalid or unsupported sizes.
 */
size_t kvc_decode_multi_workspace_bytes(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, int max_seq_len,
                                        int window, long long pool_tokens, int split_tokens);
int kvc_decode_multi_split_tokens(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, int max_seq_len,
                                  int window, long long pool_tokens, int split_tokens);

/*
 * kvc_decode_attn_multi - the attention of the n new tokens of every sequence
 * (after kvc_append_multi) over a contiguous cache (block_table == NULL) or a
 * paged one, with an optional window (>= 0).  Other arguments as for
 * kvc_decode_attn[_paged]; max_seq_len bounds seq_lens.
 */
kvc_status kvc_decode_attn_multi(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, const void* q,
                                 const void* k_cache, const void* v_cache, int T_max, const int32_t* block_table,
                                 int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* seq_lens,
                                 int max_seq_len, int window, float scale, void* out, int split_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Quantized cache (uint8 codes).  Each cached key or value vector (one
 * sequence, KV head and token) is d uint8 codes c plus a float32 pair
 * (step, zero point) = sz[.., 0:2], and stands for the values
 * (c - zero point) * step.  Contiguous: codes [B, H_kv, T_max, d], pairs
 * [B, H_kv, T_max, 2]; paged: codes [num_blocks, H_kv, block_size, d], pairs
 * [num_blocks, H_kv, block_size, 2], through the block table as above.  Half
 * the bytes of a bf16 cache per token plus 16 bytes per token and KV head.
 */

/*
 * kvc_append_u8 - kvc_append for a quantized cache.  The key is rotated as in
 * kvc_append (float32, one rounding per operation) and quantized from that
 * float32 result, the value from its dtype converted to float32, following
 * the QuantizedKVCache listing with one pair per vector, in float32 with one
 * rounding per operation and round-to-nearest-even:
 *     step = (max - min) / 255   (taken as 1 when it is 0)
 *     zero point = clamp(round(-min / step), 0, 255)
 *     code = clamp(round(x / step + zero point), 0, 255)
 * over the d elements of the vector.  q_inout (if not NULL) is rotated in
 * place exactly as kvc_append does.  dtype is that of k_new, v_new and q_inout
 * (KVC_BF16 or KVC_F32); d even and <= 256.  Position and table rules as for
 * kvc_append.
 */
kvc_status kvc_append_u8(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                         void* k_codes, float* k_sz, void* v_codes, float* v_sz, int T_max,
                         const int32_t* block_table, int block_size, int max_blocks_per_seq,
                         int num_blocks, const int32_t* positions,
                         const void* k_new, const void* v_new, void* q_inout,
                         const float* rope_cos, const float* rope_sin, int rope_rows,
                         int rope_style, void* stream);

/*
 * kvc_decode_attn_u8 - kvc_decode_attn over a quantized contiguous cache: the
 * same attention, each cached vector taken as (c - zero point) * step.  q and
 * out are bf16 [B, H_q, d]; head_dim 64 or 128; H_q / H_kv <= 32.  Workspace
 * and split rules as for kvc_decode_attn, with kvc_decode_workspace_bytes /
 * kvc_decode_split_tokens called with dtype KVC_U8.
 */
kvc_status kvc_decode_attn_u8(int B, int H_q, int H_kv, int d, const void* q, const void* k_codes,
                              const float* k_sz, const void* v_codes, const float* v_sz, int T_max,
                              const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                              int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_attn_paged_u8 - the same over quantized pools.  Requires
 * block_size a multiple of 16, split_tokens (when given) a multiple of 16, and
 * splits spanning at most 1022 blocks (KVC_ERR_UNSUPPORTED otherwise).
 */
kvc_status kvc_decode_attn_paged_u8(int B, int H_q, int H_kv, int d, const void* q, const void* k_codes,
                                    const float* k_sz, const void* v_codes, const float* v_sz, int num_blocks,
                                    int block_size, const int32_t* block_table, int max_blocks_per_seq,
                                    const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                                    int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_step_u8 - kvc_append_u8 then kvc_decode_attn_u8 (block_table
 * NULL) or kvc_decode_attn_paged_u8 in one launch over a quantized cache: the
 * decode step of kvc_decode_step with the new key and value stored as codes
 * and pairs (quantized exactly as kvc_append_u8 does) and attended from those.
 * q is the raw bf16 query (left unchanged); its rotation (kvc_append's, bf16)
 * goes to q_rot_out.  Sequence b attends positions[b] + 1 tokens (0 when the
 * position is outside the cache or the rotation table, and nothing is then
 * stored).  Sizes, layouts, workspace and split rules as for kvc_decode_step
 * and kvc_decode_attn[_paged]_u8 (kvc_decode_workspace_bytes /
 * kvc_decode_split_tokens with dtype KVC_U8); T_max is ignored when
 * block_table is given.  The results, codes and pairs are bit for bit those of
 * the two calls with the same split length.
 */
kvc_status kvc_decode_step_u8(int B, int H_q, int H_kv, int d, const void* q, void* q_rot_out, void* k_codes,
                              float* k_sz, void* v_codes, float* v_sz, int T_max, const int32_t* block_table,
                              int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* positions,
                              const void* k_new, const void* v_new, const float* rope_cos, const float* rope_sin,
                              int rope_rows, int rope_style, int max_seq_len, float scale, void* out,
                              int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 KV cache: one byte per cached element, the FP8 / INT8 quantized cache of
 * "Arsitektur Inferensi LLM" (tveniu.com), section 2 (one byte per element of
 * a GQA-8 cache), whose section 8 starts an engine with an "fp8" KV-cache
 * dtype; "KV Cache 최적화 심층 분석" (youngju.dev) turns on fp8_e5m2 in its vLLM
 * commands.  The pages leave the format open; these calls read it as the OCP
 * 8-bit floating-point formats:
 *   KVC_FP8_E4M3  sign, 4 exponent bits (bias 7), 3 mantissa bits, largest
 *                 finite 448, no infinities; each cached vector gets the
 *                 float32 scale (largest magnitude of its d elements) / 448
 *                 (1 when that is 0) and stores the codes of x / scale;
 *   KVC_FP8_E5M2  sign, 5 exponent bits (bias 15), 2 mantissa bits, largest
 *                 finite 57344; the direct cast (scale 1).
 * Codes round to nearest, ties to even, from float32 (one rounding for the
 * division, one for the code), saturating at the largest finite value.  The
 * layout is the uint8 cache's: codes uint8 [B, H_kv, T_max, d] (or pools
 * [num_blocks, H_kv, block_size, d]) and float32 pairs [..., 2] = (scale, 0),
 * so a cached value reads back as decode(code) * scale.  The key is rotated
 * as in kvc_append (float32) and quantized from that float32 result, the value
 * from its dtype converted to float32.  Attention, sizes, rules and errors are
 * those of the *_u8 calls with the same arguments (format first); the sizing
 * queries take the format as their dtype.  A format other than the two is
 * KVC_ERR_UNSUPPORTED.
 */
kvc_status kvc_append_fp8(kvc_dtype format, kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                          void* k_codes, float* k_sz, void* v_codes, float* v_sz, int T_max,
                          const int32_t* block_table, int block_size, int max_blocks_per_seq,
                          int num_blocks, const int32_t* positions,
                          const void* k_new, const void* v_new, void* q_inout,
                          const float* rope_cos, const float* rope_sin, int rope_rows,
                          int rope_style, void* stream);

kvc_status kvc_decode_attn_fp8(kvc_dtype format, int B, int H_q, int H_kv, int d, const void* q,
                               const void* k_codes, const float* k_sz, const void* v_codes, const float* v_sz,
                               int T_max, const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                               int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

kvc_status kvc_decode_attn_paged_fp8(kvc_dtype format, int B, int H_q, int H_kv, int d, const void* q,
                                     const void* k_codes, const float* k_sz, const void* v_codes,
                                     const float* v_sz, int num_blocks, int block_size, const int32_t* block_table,
                                     int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, float scale,
                                     void* out, int split_tokens, void* workspace, size_t workspace_bytes,
                                     void* stream);

kvc_status kvc_decode_step_fp8(kvc_dtype format, int B, int H_q, int H_kv, int d, const void* q, void* q_rot_out,
                               void* k_codes, float* k_sz, void* v_codes, float* v_sz, int T_max,
                               const int32_t* block_table, int block_size, int max_blocks_per_seq, int num_blocks,
                               const int32_t* positions, const void* k_new, const void* v_new,
                               const float* rope_cos, const float* rope_sin, int rope_rows, int rope_style,
                               int max_seq_len, float scale, void* out, int split_tokens, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Latent cache (multi-head latent attention), following the
 * MultiHeadLatentAttention listing of "KV Cache 최적화 심층 분석: GQA·MLA·MHA
 * 어텐션 메커니즘과 메모리 효율화 전략" (youngju.dev).  Each token is cached as
 * one row of d_latent + rope_dim values, [c_kv | k_rope]; the cache is
 * [B, T_max, d_latent + rope_dim] (one layer; the listing's (c_kv, k_rope)
 * pair packed along the last axis).  Head h's key and value of token t are
 * the up-projections of its latent:
 *     k_h,t = W_uk[h*d_k : (h+1)*d_k, :] c_t + b_uk[h*d_k : (h+1)*d_k]
 *     v_h,t = W_uv[h*d_k : (h+1)*d_k, :] c_t + b_uv[h*d_k : (h+1)*d_k]
 * (W [n_heads * d_k, d_latent] and b [n_heads * d_k], nn.Linear's layout),
 * and out_h = softmax(q_h . k_h,t * scale) v_h over the attended tokens.  As
 * in the listing, k_rope is stored but not attended.  bf16 only.
 *
 * The library computes this in the absorbed form, an exact rewrite:
 *     scores  q~_h . c_t * scale with q~_h = W_uk,h^T q_h (the key bias adds
 *             q_h . b_uk,h to every score of head h, which the softmax removes,
 *             so it is not an argument);
 *     out_h = W_uv,h (sum_t p_t c_t) + b_uv,h      (the weights p_t sum to 1),
 * so the cache is read once, as d_latent values per token, for all heads.
 */

/*
 * kvc_append_mla - store the new token's row [c_kv_new[b] | k_rope_new[b]]
 * (bit copies, nothing rotated: the listing rotates neither) at slot
 * positions[b] of sequence b.  c_kv_new [B, d_latent], k_rope_new
 * [B, rope_dim] (NULL when rope_dim == 0), dtype KVC_BF16 or KVC_F32 (of
 * every buffer).  d_latent + rope_dim must be a multiple of 8 (16-byte rows
 * in bf16).  A position outside [0, T_max) writes nothing.
 */
kvc_status kvc_append_mla(kvc_dtype dtype, int B, int d_latent, int rope_dim, void* cache, int T_max,
                          const int32_t* positions, const void* c_kv_new, const void* k_rope_new, void* stream);

/*
 * Workspace bytes (256-byte aligned) and split length of kvc_decode_attn_mla
 * with these sizes (max_seq_len bounds the attended lengths; split_tokens 0 =
 * the library's choice, else a multiple of 32).  (size_t)-1 / -1 for invalid
 * or unsupported sizes.  Past the first kvc_workspace_zeroed_bytes() bytes,
 * which these calls neither read nor write (so one buffer can serve them and
 * the other decode calls), the workspace holds the absorbed queries and the
 * merged latent context, [B, H, d_latent] float32 each, and the split
 * partials, [B, H, splits] (max, sum) pairs and [B, H, splits, d_latent]
 * float32; none of it needs initialisation.
 */
size_t kvc_decode_mla_workspace_bytes(int B, int H, int d_latent, int max_seq_len, int split_tokens);
int kvc_decode_mla_split_tokens(int B, int H, int d_latent, int max_seq_len, int split_tokens);

/*
 * kvc_decode_attn_mla - attention of one new query per sequence over the
 * first seq_lens[b] tokens of its latent cache.
 *   q      bf16 [B, H, d_k]          query heads (d_k a multiple of 32, <= 512)
 *   cache  bf16 [B, T_max, d_latent + rope_dim], d_latent 128, 256 or 512
 *   w_uk, w_uv  bf16 [H * d_k, d_latent];  b_uv bf16 [H * d_k] or NULL (zero)
 *   scale  <= 0: 1 / sqrt(d_k)
 *   out    float32 [B, H, d_k]  (float32: the result of the value
 *          up-projection, before any rounding to a storage type)
 * seq_lens[b] in [0, max_seq_len], max_seq_len <= T_max; a sequence of length
 * 0 gives zeros.  Four launches: absorbed queries, the streaming pass over
 * the cache (one workgroup per sequence, 32-head chunk and token split), the
 * merge of the splits, the value up-projection.
 */
kvc_status kvc_decode_attn_mla(int B, int H, int d_k, int d_latent, int rope_dim, const void* q,
                               const void* cache, int T_max, const int32_t* seq_lens, int max_seq_len,
                               const void* w_uk, const void* w_uv, const void* b_uv, float scale, float* out,
                               int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_decode_step_mla - kvc_append_mla then kvc_decode_attn_mla in one call:
 * the new row is stored at slot positions[b] and sequence b attends
 * positions[b] + 1 tokens (0 when the position is outside [0, T_max)).
 * max_seq_len bounds positions[b] + 1.  The append rides in the first launch.
 */
kvc_status kvc_decode_step_mla(int B, int H, int d_k, int d_latent, int rope_dim, const void* q, void* cache,
                               int T_max, const int32_t* positions, const void* c_kv_new,
                               const void* k_rope_new, int max_seq_len, const void* w_uk, const void* w_uv,
                               const void* b_uv, float scale, float* out, int split_tokens, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
