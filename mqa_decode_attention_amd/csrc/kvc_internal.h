// kvc_internal.h - parameter blocks and launchers shared by the C ABI layer
// (kvc_api.hip) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

// Codes of the 8-bit caches (the cache's dtype: KVC_U8, KVC_FP8_E4M3,
// KVC_FP8_E5M2).
constexpr int kQ8Affine = 0;   // uint8 codes on an affine grid, (step, zero point) per vector
constexpr int kQ8E4M3 = 1;     // OCP FP8 E4M3 codes, (scale, 0) per vector
constexpr int kQ8E5M2 = 2;     // OCP FP8 E5M2 codes, (1, 0) per vector

struct AppendParams {
    kvc_dtype dtype;
    int B, H_q, H_kv, d;
    void* k_cache;
    void* v_cache;
    int T_max;                   // contiguous capacity (tokens)
    const int32_t* block_table;  // NULL => contiguous
    int block_size, max_blocks_per_seq, num_blocks;
    int capacity;                // tokens addressable per sequence
    const int32_t* positions;
    const void* k_new;
    const void* v_new;
    void* q_inout;
    const void* q_in;            // NULL: q_inout is rotated in place; else read from here, rotated into q_inout
    const float* rope_cos;
    const float* rope_sin;
    int rope_rows;
    int rope_style;
    int ring;                    // contiguous ring of T_max slots: position p -> slot p % T_max
    int qlen;                    // new tokens per sequence (token i at position positions[b] + i; 0 means 1)
    // 8-bit cache (launch_append_u8): k_cache / v_cache hold the codes
    // [.., d] and these the float pair of each vector - (step, zero point) of
    // the uint8 grid, or (scale, 0) of the FP8 formats (qfmt: kQ8Affine,
    // kQ8E4M3, kQ8E5M2)
    float* k_sz;
    float* v_sz;
    int qfmt;
};

hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_append_u8(const AppendParams& p, hipStream_t stream);

// Split-decode launch plan, a pure function of the sizes (no device query), so
// that kvc_decode_workspace_bytes and the decode call always agree.
struct DecodePlan {
    bool mfma;          // matrix-core kernel (bf16) rather than the vector kernel
    int heads_per_wg;   // query heads one workgroup serves (a divisor of G)
    int n_chunks;       // G / heads_per_wg
    int split_tokens;   // tokens per split
    int split_tail;     // the last split of a sequence takes up to this many tokens more
    int n_splits;       // splits of the longest sequence (>= 1)
    size_t ws_ml;       // byte offsets inside the workspace
    size_t ws_part;
    size_t ws_bytes;    // 0 when n_splits == 1
    bool merge_in_kernel;   // the streaming kernel merges the splits (no merge launch)
    bool one_round;     // every workgroup of the split plan fits on the device at once
    // Compacted schedule (bf16 matrix-core kernel, contiguous cache, one new
    // token, library splits, plans of several rounds): the kernel picks the
    // split length, at least split_tokens, from the lengths so that the
    // splits fit in cmp_slots workgroups, and merges them itself.
    bool compact;
    int cmp_slots, cmp_step, cmp_tmax;
    size_t ws_nsp;      // byte offset of its per-unit split counts in the workspace
    // Balanced schedule of the bf16 matrix-core kernel: bal_wg workgroups share
    // the steps of all units equally, whatever the lengths (ws_ml / ws_part
    // then hold 2 * G partial rows per workgroup; ws_bytes also covers the
    // split layout, which calls the balanced kernel does not serve use).
    bool bal;
    int bal_wg;
};

// Sequences the compacted numbering handles (64 lengths per lane load).
constexpr int kCmpChunks = 4;
constexpr int kCmpMaxB = 64 * kCmpChunks;

// Sequences the balanced schedule handles (their lengths are staged in LDS).
constexpr int kBalMaxB = 512;
// Most tokens one workgroup of the balanced schedule takes (its paged
// segments then span at most 960 + 2 blocks of 16 tokens, inside the kTblMax
// entries of the staged table): 240 loop steps of the bf16 kernel, 120 of the
// quantized one.
constexpr int kBalMaxTokens = 15360;

// Largest split count the merge step supports (partials live in LDS).
constexpr int kMaxSplits = 256;

// Every decode and latent-cache workspace starts with kMergeCounters 32-bit
// arrival counters, one per (sequence, KV head, chunk) unit: the matrix-core
// kernel's splits count themselves in, and the last one to arrive merges the
// unit's partial results (no separate merge launch).  The counters must be
// zero before a workspace is first used; the last arrival's increment wraps
// its counter back to zero, so every completed call leaves them zero.  Only
// plans of one round of workgroups merge so (see plan_decode); the others,
// and plans with more units, merge in a separate launch.
constexpr int kMergeCounters = 16384;
constexpr size_t kWsCounterBytes = kMergeCounters * sizeof(unsigned);

// Block-table entries of one split that the paged kernels with staged tiles
// keep in LDS (4 KiB).  The bf16 kernel falls back to per-group table reads
// for splits spanning more blocks; the quantized one needs splits within it.
constexpr int kTblMax = 1024;


struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const int32_t* seq_lens;
    const int32_t* block_table;  // NULL => contiguous
    float* ws_part;              // [B*H_q, n_splits, d]   weighted-value partials
    float2* ws_ml;               // [B*H_q, n_splits]      (running max (log2), sum)
    unsigned* merge_cnt;         // [units] arrival counters (in-kernel merge), or NULL
    int B, H_q, H_kv, G, n_chunks;
    int T_max, block_size, max_blocks_per_seq, num_blocks;
    int max_seq_len, split_tokens, n_splits;
    int split_tail;              // the last split also takes up to this many tokens (a short remainder)
    int n_wg, n_wg_pad;          // logical workgroups, padded to a multiple of 8
    int bal;                     // balanced schedule (n_wg workgroups share all units' steps)
    int compact;                 // compacted schedule: split length from the lengths, existing splits first
    int* ws_nsp;                 // [B * H_kv] its split count per unit, for the merge kernel
    int cmp_slots, cmp_step, cmp_tmax;   // its workgroup budget, loop step, longest split
    float scale_log2;            // softmax scale * log2(e)

    // Set for kvc_decode_step: lengths come from positions (L_b = positions[b] + 1)
    // and, in the fused kernel, the append happens inside the streaming pass.
    const int32_t* positions;    // [B] slot of the new token, or NULL
    const void* k_new;           // [B, H_kv, d] raw key / value of the new token
    const void* v_new;
    const void* q_raw;           // [B, H_q, d] unrotated query (fused kernel)
    void* q_rot_out;             // [B, H_q, d] receives the rotated query
    const float* rope_cos;       // [rope_rows, d/2]
    const float* rope_sin;
    int rope_rows, rope_style;
    int capacity;                // tokens addressable per sequence
    int valu_step;               // the vector kernel does the step's append itself (contiguous cache)

    // Sliding window: a sequence holding L tokens attends [max(0, L - window), L)
    // (window 0: all of them); ring: the cache is a ring of T_max slots (token t
    // in slot t % T_max) and the slots [0, min(L, T_max)) are attended.
    int window, ring;
    int align;                   // split origins are multiples of this (a power of two)

    // New tokens per sequence (1 for a single-token step).  With qlen > 1, q
    // and out are [B, qlen, H_q, d] and query token i of a sequence holding L
    // tokens attends [.., L - qlen + i + 1) (causal among the new tokens); the
    // G * qlen query rows of a KV group are cut into n_chunks chunks.
    int qlen;
};

// Attended length of sequence b: from positions (a decode step, after its
// append) or from seq_lens; clamped to [0, max_seq_len].  A step whose slot is
// outside the cache or the rotation table attends over nothing.
__device__ __forceinline__ int len_from_position(const DecodeParams& p, int pos) {
    const int L = (pos >= 0 && pos < p.capacity && pos < p.rope_rows) ? pos + 1 : 0;
    return L > p.max_seq_len ? p.max_seq_len : L;
}

__device__ __forceinline__ int attended_len(const DecodeParams& p, int b) {
    if (p.positions) return len_from_position(p, p.positions[b]);
    const int L = p.seq_lens[b];
    return L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
}

// Tokens a decode of a sequence holding L tokens attends, [lo, hi), and the
// origin org of its splits: split s covers [org + s * split_tokens, ...) up to
// hi, the last one to hi (a remainder of up to split_tail tokens joins it).  org is lo rounded down to p.align (16 for the paged kernels, whose tiles
// are 16-row groups of one block); those kernels mask the rows in [org, lo)
// and do not read them.
struct TokenRange {
    int lo, hi, org;
};
__device__ __forceinline__ TokenRange token_range(const DecodeParams& p, int L) {
    TokenRange r;
    if (p.ring) {
        r.lo = 0;
        r.hi = L < p.T_max ? L : p.T_max;
    } else {
        // (with several new tokens the first one's window starts earliest)
        const int first_hi = L - p.qlen + 1;
        r.hi = L;
        r.lo = (p.window > 0 && first_hi > p.window) ? first_hi - p.window : 0;
    }
    r.org = r.lo & ~(p.align - 1);
    return r;
}
// Splits of that range (at least 1).
__device__ __forceinline__ int split_count(const DecodeParams& p, const TokenRange& r) {
    const int n = (r.hi - r.org - p.split_tail + p.split_tokens - 1) / p.split_tokens;
    return n < 1 ? 1 : n;
}
// End of split s of nsp (exclusive).
__device__ __forceinline__ int split_end(const DecodeParams& p, const TokenRange& r, int s, int nsp) {
    const int e = r.org + (s + 1) * p.split_tokens;
    return (s == nsp - 1 || e > r.hi) ? r.hi : e;
}

// ---------------------------------------------------------------------------
// Compacted schedule of the bf16 streaming kernel over a contiguous cache
// (plans that would take several rounds of workgroups).  The host knows only
// the longest sequence, so its split plan leaves many splits past the end of
// shorter ones, and a split that exists competes for a slot with those that
// do not.  Here every workgroup reads all lengths (up to kCmpMaxB, 64 per
// load, requested together) and picks the split length T itself: the
// shortest multiple of the loop step, at least the host's split_tokens, whose
// splits of all units (H_kv * nsp_b per sequence) fit in cmp_slots
// workgroups - one round, so every split starts at once.  The splits that
// exist, counted in unit order, then take workgroup indices 0, 1, ...; the
// rest exit at once.  Every workgroup computes the same T and counts from
// the same lengths; the first split of each unit records the unit's split
// count in the workspace (ws_nsp) for the merge kernel.
// ---------------------------------------------------------------------------

struct CmpSeg {
    int unit, split, nsp;   // b * H_kv + j, this split, the unit's splits
    int L, pos;             // attended length, new-token slot (FUSED)
    int T;                  // split length
};

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Splits of a sequence of L tokens at split length T (split_count's rule).
__device__ __forceinline__ int cmp_splits(const DecodeParams& p, int L, int T) {
    const TokenRange r = token_range(p, L);
    const int n = (r.hi - r.org - p.split_tail + T - 1) / T;
    return n < 1 ? 1 : n;
}

// Lengths (and, FUSED, new-token slots) of sequences 64 k + lane.
template <bool FUSED>
__device__ __forceinline__ void cmp_lengths(const DecodeParams& p, int (&lens)[kCmpChunks],
                                            int (&poss)[kCmpChunks]) {
    const int ln = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kCmpChunks; ++k) {
        const int bb = 64 * k + ln;
        poss[k] = 0;
        lens[k] = 0;
        if (bb < p.B) {
            if constexpr (FUSED) {
                poss[k] = p.positions[bb];
                lens[k] = len_from_position(p, poss[k]);
            } else {
                lens[k] = attended_len(p, bb);
            }
        }
    }
}

// The unit and split of workgroup wid (false: it takes none).  The split
// length T: a first estimate from the tokens the splits cover, over the slots
// less half a split per unit (a sequence's last split is on average half
// full); then, while the units' splits (counted by the same prefix sum over
// the lanes that locates wid) exceed the slots, longer: twice in proportion
// to the count's excess, then in proportion to the splits beyond each unit's
// first (those that shrink with T), which always ends within the passes
// (modelled on the host over random ragged shapes: never over the slots, at
// most ~8 % longer than the shortest length that fits; mostly one pass).  T
// never passes cmp_tmax, one split per sequence.
template <bool FUSED>
__device__ __forceinline__ bool cmp_locate(const DecodeParams& p, int wid, CmpSeg& c) {
    const int ln = threadIdx.x & 63;
    int lens[kCmpChunks], poss[kCmpChunks];
    cmp_lengths<FUSED>(p, lens, poss);
    // (the estimate in float32: only a starting point, which the count below
    // checks; the butterfly sum has a fixed order, so every workgroup gets
    // the same value)
    float span = 0.0f;
#pragma unroll
    for (int k = 0; k < kCmpChunks; ++k) {
        if (64 * k + ln < p.B) {
            const TokenRange r = token_range(p, lens[k]);
            span += static_cast<float>(r.hi - r.org);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) span += __shfl_xor(span, o, 64);
    const int step = p.cmp_step;
    const int units = p.B * p.H_kv;
    const float room = static_cast<float>(max(1, p.cmp_slots - units / 2));
    const float steps = ceilf(span * static_cast<float>(p.H_kv) / (room * static_cast<float>(step)));
    int T = steps >= static_cast<float>(p.cmp_tmax / step) ? p.cmp_tmax : static_cast<int>(steps) * step;
    T = __builtin_amdgcn_readfirstlane(max(T, p.split_tokens));
    // per chunk: the lane's splits (H_kv * nsp_b), their inclusive prefix over
    // the lanes, and the chunk's total
    int n[kCmpChunks], inc[kCmpChunks], tot[kCmpChunks];
    for (int pass = 0;; ++pass) {
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kCmpChunks; ++k) {
            n[k] = inc[k] = tot[k] = 0;
            if (64 * k >= p.B) continue;
            n[k] = 64 * k + ln < p.B ? cmp_splits(p, lens[k], T) * p.H_kv : 0;
            inc[k] = n[k];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(inc[k], o, 64);
                if (ln >= o) inc[k] += v;
            }
            tot[k] = __shfl(inc[k], 63, 64);
            cnt += tot[k];
        }
        if (cnt <= p.cmp_slots || T >= p.cmp_tmax || pass == 5) break;
        const long long free_slots = max(1, p.cmp_slots - units);
        const long long grown = pass < 2 ? static_cast<long long>(T) * cnt / p.cmp_slots
                                         : (static_cast<long long>(T) * (cnt - units) + free_slots - 1) / free_slots;
        T = static_cast<int>(min<long long>(max<long long>(T + step, (grown + step - 1) / step * step), p.cmp_tmax));
        T = __builtin_amdgcn_readfirstlane(T);
    }
    int before = 0;                       // splits of the sequences of earlier chunks
    bool found = false;
    c = CmpSeg{};
    c.T = T;
#pragma unroll
    for (int k = 0; k < kCmpChunks; ++k) {
        if (!found && wid < before + tot[k]) {
            // the first lane whose prefix passes wid
            const int lk = __builtin_ctzll(__ballot(before + inc[k] > wid));
            const int nk = __shfl(n[k], lk, 64);
            const int r = wid - before - (__shfl(inc[k], lk, 64) - nk);   // index among the sequence's splits
            c.L = __shfl(lens[k], lk, 64);
            c.pos = __shfl(poss[k], lk, 64);
            c.nsp = nk / p.H_kv;
            c.unit = (64 * k + lk) * p.H_kv + r / c.nsp;
            c.split = r % c.nsp;
            found = true;
        }
        before += tot[k];
    }
    c.unit = __builtin_amdgcn_readfirstlane(c.unit);
    c.split = __builtin_amdgcn_readfirstlane(c.split);
    c.nsp = __builtin_amdgcn_readfirstlane(c.nsp);
    c.L = __builtin_amdgcn_readfirstlane(c.L);
    c.pos = __builtin_amdgcn_readfirstlane(c.pos);
    return found;
}

// Returns false (and leaves *plan untouched) when the sizes cannot be planned.
// pool_tokens: token capacity of a paged pool (num_blocks * block_size), which
// bounds the tokens all sequences attend over together; 0 for a contiguous cache.
// qlen: new tokens per sequence (query rows G * qlen per KV group).
// allow_bal: the call may use the balanced schedule (a single-token decode
// over a full cache); the workspace size is the same either way.
bool plan_decode(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                 long long pool_tokens, int split_tokens, DecodePlan* plan, const char** why, int qlen = 1,
                 bool allow_bal = true);

// Is there a kernel for this (dtype, head dim, heads per workgroup)?
bool decode_supported(kvc_dtype dtype, int d, int heads_per_wg);

// Tokens one workgroup consumes per pass of all its waves (split sizes are a
// multiple of this unless the caller fixes them).
int decode_tile_tokens(kvc_dtype dtype, int d);

// Optional events recorded by the command processor exactly around one kernel.
struct KernelTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

template <typename Kernel, typename... Args>
inline hipError_t launch_timed(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream,
                               const KernelTiming& tm, const Args&... args) {
    if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, tm.start, tm.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
    return hipGetLastError();
}

// The streaming kernel: one workgroup per (sequence, KV head, chunk, split).
hipError_t launch_decode_split(kvc_dtype dtype, int d, int heads_per_wg, bool paged,
                               const DecodeParams& p, hipStream_t stream, const KernelTiming& tm);

// The matrix-core streaming kernel (bf16; head_dim 64/128/256; G <= 32): one
// workgroup per (sequence, KV head, split) serves all G query heads.
bool decode_mfma_supported(kvc_dtype dtype, int d, int G);
// Tokens one workgroup of that kernel covers per loop step (four waves'
// tiles); splits of a whole number of steps stream fastest.
int decode_mfma_step_tokens(int d, bool paged);
// Workgroups of the MFMA decode kernel one compute unit holds at once (set by
// its registers and LDS at this head dim, group size and cache layout).
int decode_mfma_wgs_per_cu(int d, int G, bool paged);
// rows: query rows per workgroup (G; with several new tokens, up to 32 of the
// G * qlen rows, multi = true).
hipError_t launch_decode_mfma(int d, int rows, bool paged, bool fused, bool multi, const DecodeParams& p,
                              hipStream_t stream, const KernelTiming& tm);

// The matrix-core streaming kernel over an 8-bit cache (bf16 q and out;
// head_dim 64/128; G <= 32); k_sz / v_sz hold the pair of each cached vector:
// (step, zero point) of uint8 codes, (scale, 0) of FP8 codes (qfmt:
// kQ8Affine, kQ8E4M3, kQ8E5M2).
bool decode_u8_supported(int d, int G);
int decode_u8_step_tokens();
int decode_u8_wgs_per_cu(int d, int G);
// fused: the step's append runs inside (p.positions etc. set; the new token's
// codes and pairs are written to the cache and k_sz / v_sz).
hipError_t launch_decode_u8(int d, int G, bool paged, bool fused, int qfmt, const DecodeParams& p, float* k_sz,
                            float* v_sz, hipStream_t stream, const KernelTiming& tm);

// The log-sum-exp merge of the splits (only when n_splits > 1).
hipError_t launch_decode_merge(kvc_dtype dtype, int d, const DecodeParams& p, hipStream_t stream);

// ---------------------------------------------------------------------------
// Latent cache (multi-head latent attention), absorbed form.
// ---------------------------------------------------------------------------

struct MlaParams {
    const void* q;               // bf16 [B, H, d_k]
    void* cache;                 // bf16 [B, T_max, row], row = d_latent + rope_dim
    const int32_t* seq_lens;     // [B] attended lengths, or NULL when positions is set
    const int32_t* positions;    // step: the new row goes to slot positions[b], L = positions[b] + 1
    const void* c_new;           // step: [B, d_latent] new latent (NULL: no append)
    const void* r_new;           // step: [B, rope_dim] new rope part (NULL when rope_dim == 0)
    const void* w_uk;            // bf16 [H * d_k, d_latent]
    const void* w_uv;            // bf16 [H * d_k, d_latent]
    const void* b_uv;            // bf16 [H * d_k] or NULL
    float* out;                  // [B, H, d_k]
    float* qt;                   // absorbed queries times the scale as bf16 hi + lo planes, [2][B, H, d_latent] (workspace)
    float* ctx;                  // [B, H, d_latent] softmax-weighted latents (workspace)
    float2* ws_ml;               // [B * H, n_splits] (running max (log2), sum)
    float* ws_part;              // [B * H, n_splits, d_latent]
    int B, H, d_k, d_latent, rope_dim, row, T_max, max_seq_len;
    int split_tokens, n_splits, n_chunks, n_wg;
    float scale_log2;
};

struct MlaPlan {
    int split_tokens, n_splits, n_chunks;
    size_t qt, ctx, ws_ml, ws_part, ws_bytes;   // byte offsets / total
};

// Tokens of one tile of the latent-cache kernel (split lengths are multiples).
constexpr int kMlaTile = 32;
// Query heads one workgroup of that kernel serves (larger H: several chunks).
constexpr int kMlaHeads = 32;

bool plan_mla(int B, int H, int d_latent, int max_seq_len, int split_tokens, MlaPlan* plan, const char** why);

// Bit copy of the new rows [c_kv | k_rope] into a latent cache (elem_bytes 2 or 4).
hipError_t launch_append_mla(int elem_bytes, int B, int d_latent, int rope_dim, void* cache, int T_max,
                             const int32_t* positions, const void* c_new, const void* r_new, hipStream_t stream);

// The four launches of a latent-cache decode (the append rides in the first
// when p.c_new is set); tm times the streaming kernel.
hipError_t launch_mla(const MlaParams& p, hipStream_t stream, const KernelTiming& tm);

// Streaming-read probe (kvc_hbm_read_probe).
hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, int workgroups,
                             bool nontemporal, hipStream_t stream);

}  // namespace kvc
