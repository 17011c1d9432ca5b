// kvc_api.hip - the C ABI of libkvc (declared in include/kvc.h): argument
// checks, launch planning and error reporting around the kernels.
//
// Every check here runs on the host before any HIP call, so a bad call returns
// its status without touching the device.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kvc_internal.h"

namespace {

// The 8-bit caches: their dtype codes, and the code format of each.
bool is_q8(kvc_dtype dt) { return dt == KVC_U8 || dt == KVC_FP8_E4M3 || dt == KVC_FP8_E5M2; }
int q8_format(kvc_dtype dt) {
    return dt == KVC_FP8_E4M3 ? kvc::kQ8E4M3 : (dt == KVC_FP8_E5M2 ? kvc::kQ8E5M2 : kvc::kQ8Affine);
}

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_prof_start = nullptr;   // one-shot timing events (kvc_profile_next_decode)
thread_local hipEvent_t g_prof_stop = nullptr;

kvc_status fail(kvc_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

kvc_status fail(kvc_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

kvc_status ok() {
    g_last_error[0] = '\0';
    return KVC_OK;
}

kvc_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_bytes(kvc_dtype dt) { return dt == KVC_BF16 ? 2 : 4; }

bool dtype_ok(kvc_dtype dt) { return dt == KVC_BF16 || dt == KVC_F32; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Heads of one group served by one workgroup: the largest of 8, 4, 2, 1 that
// divides G (larger groups are served in several chunks).
int heads_per_wg(int G) {
    for (int c : {8, 4, 2, 1})
        if (G % c == 0) return c;
    return 1;
}

// Workgroups the split heuristic of the VALU kernel aims for: four per
// compute unit of an MI355X.
constexpr int kTargetWorkgroups = 4 * 256;

// Compute units of the current device (256 on an MI355X, also the answer
// when no device can be queried, e.g. when sizing a workspace on a host
// without a GPU).  Cached per device.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Common checks of the head/group sizes.
kvc_status check_heads(kvc_dtype dt, int B, int H_q, int H_kv, int d) {
    if (!dtype_ok(dt)) return fail(KVC_ERR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dt));
    if (B < 0 || H_q <= 0 || H_kv <= 0 || d <= 0)
        return fail(KVC_ERR_SHAPE, "sizes must be positive (B=%d H_q=%d H_kv=%d d=%d)", B, H_q, H_kv, d);
    if (H_q % H_kv != 0)
        return fail(KVC_ERR_SHAPE, "H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
    return KVC_OK;
}

}  // namespace

namespace kvc {

bool plan_decode(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                 long long pool_tokens, int split_tokens, DecodePlan* plan, const char** why, int qlen,
                 bool allow_bal) {
    DecodePlan pl{};
    const int G = H_q / H_kv;
    if (qlen > 1 && (dtype != KVC_BF16 || !decode_mfma_supported(dtype, d, 1))) {
        *why = "several new tokens per sequence need bf16 and head_dim 64, 128 or 256";
        return false;
    }
    const bool u8 = is_q8(dtype);         // 8-bit cache: its own matrix-core kernel
    if (u8 && !decode_u8_supported(d, G)) {
        *why = "the quantized-cache kernel needs head_dim 64 or 128 and H_q / H_kv <= 32";
        return false;
    }
    pl.mfma = u8 || decode_mfma_supported(dtype, d, G);
    // query rows of a KV group: G, or G * qlen for several new tokens, served
    // in chunks of 16 or 32 rows (one or two 16-row head blocks)
    const int rows = G * std::max(qlen, 1);
    if (qlen > 1) {
        pl.heads_per_wg = rows <= 16 ? rows : 32;
        pl.n_chunks = (rows + pl.heads_per_wg - 1) / pl.heads_per_wg;
        pl.heads_per_wg = std::min(rows, pl.heads_per_wg);
    } else {
        pl.heads_per_wg = pl.mfma ? G : heads_per_wg(G);
        pl.n_chunks = G / pl.heads_per_wg;
    }
    if (!pl.mfma && !decode_supported(dtype, d, pl.heads_per_wg)) {
        *why = "no decode kernel for this dtype and head_dim (head_dim must be 16, 32, 64, 128 or 256)";
        return false;
    }
    const long long units = static_cast<long long>(B) * H_kv * pl.n_chunks;
    // workgroups of the streaming kernel the device holds at once
    const long long slots = static_cast<long long>(cu_count()) *
                            (u8 ? decode_u8_wgs_per_cu(d, G)
                                : (pl.mfma ? decode_mfma_wgs_per_cu(d, pl.heads_per_wg, pool_tokens > 0) : 1));
    const int tile = u8 ? decode_u8_step_tokens()
                        : (pl.mfma ? decode_mfma_step_tokens(d, pool_tokens > 0) : decode_tile_tokens(dtype, d));
    const int L = std::max(max_seq_len, 1);
    long long ts;
    int tail = 0;       // tokens the last split may take beyond split_tokens
    auto n_of = [&](long long t) { return std::max(1LL, (L - tail + t - 1) / t); };
    if (split_tokens > 0) {
        ts = split_tokens;
        if ((L + ts - 1) / ts > kMaxSplits) {
            *why = "split_tokens gives more splits than the merge step supports";
            return false;
        }
    } else if (pl.mfma) {
        // One round of workgroups that fills every compute unit equally
        // streams best: fewer leave CUs idle, a partial second round leaves
        // a tail.  A paged pool holding much less than B * L tokens means
        // ragged lengths, where about four rounds of shorter splits even out
        // the per-sequence work.  Groups of more than 16 heads (two head
        // blocks per wave, two waves per SIMD) do several times the work per
        // tile and wait on latency more than on bandwidth: about three
        // workgroups per slot (ragged 64-sequence MQA: 27 us at 384-token
        // splits, 30-31 us at one round of 1088).  Each split also writes G
        // partial rows, about G / split_tokens of the bytes it reads: at
        // least 32 * G tokens per split keeps that near 3 %, 12 * G (for
        // the large groups) near 8 %.
        const long long full = units * L;
        const int rpw = pl.heads_per_wg;      // query rows per workgroup
        const bool large_group = rpw > 16;
        if (pool_tokens > 0 && pool_tokens * H_kv * 10 < full * 9) {
            ts = (pool_tokens * H_kv + 4 * slots - 1) / (4 * slots);
        } else {
            const long long S = std::max(1LL, (large_group ? 3 : 1) * slots / std::max(1LL, units));
            ts = (L + S - 1) / S;
        }
        const long long least = (large_group ? 12LL : 32LL) * rpw;
        ts = std::max<long long>(ts, least);
        // Whole loop steps of the kernel (64 or 128 tokens): splits that
        // start off a step boundary (e.g. balanced 4112 + 4081 for 8193
        // tokens with 128-token steps) streamed 2-13 % slower.
        const long long up = (ts + tile - 1) / tile * tile;
        const long long dn = ts / tile * tile;
        ts = up;
        if (!u8 && pool_tokens == 0 && qlen <= 1) {
            // Over a contiguous cache the last split also takes a remainder
            // of less than one step: 8193 tokens are two splits of 4096 and
            // 4097 rather than 4160 and 4033 (the longest split one step
            // shorter; its extra token is the step's new one, patched in
            // from registers with no memory read), and no split of a few
            // tokens pays a whole prologue.
            tail = tile - 1;
            if (dn >= least && n_of(dn) <= n_of(up)) ts = dn;
        }
        while (n_of(ts) > kMaxSplits) ts += tile;
    } else {
        long long want = units > 0 ? (kTargetWorkgroups + units - 1) / units : 1;
        want = std::max(1LL, std::min<long long>(want, kMaxSplits));
        ts = (L + want - 1) / want;
        ts = (ts + tile - 1) / tile * tile;
        while ((L + ts - 1) / ts > kMaxSplits) ts += tile;
    }
    pl.split_tokens = static_cast<int>(std::min<long long>(ts, 0x7FFFFFFF));
    pl.split_tail = tail;
    pl.n_splits = static_cast<int>(n_of(ts));
    pl.one_round = units * pl.n_splits <= slots;
    // Compacted schedule for contiguous caches whose split plan takes several
    // rounds: the kernel picks the split length from the lengths (the
    // shortest that fits every split in one round of `slots` workgroups);
    // the host plans the shortest length it may pick, which sizes the
    // workspace, and the merge kernel derives the kernel's length again.
    // (Ragged 64-sequence MQA: the split plan's 384-token splits 25.7 us +
    // a 4 us merge launch, step 29.6 us; 640-token splits with the existing
    // splits numbered first 24.0 us, step 27.0.  Merged in the streaming
    // kernel instead, as one-round plans are, its 32-row groups took 28.4 us,
    // step 29.1: the last split of a unit merges up to 32 rows x 11 splits
    // alone, where the merge kernel spreads them over a wave per row.)
    if (allow_bal && split_tokens == 0 && pl.mfma && !u8 && pool_tokens == 0 && qlen <= 1 && !pl.one_round &&
        B <= kCmpMaxB && units * 2 <= slots) {
        // (no remainder joins a sequence's last split here: in one round the
        // longest split sets the time, and a remainder of up to a step made
        // some splits 703 tokens long instead of 640 - 25.3 against 24.0 us)
        const long long least = (pl.heads_per_wg > 16 ? 12LL : 32LL) * pl.heads_per_wg;
        tail = 0;
        ts = std::max<long long>(tile, (least + tile - 1) / tile * tile);
        while (n_of(ts) > kMaxSplits) ts += tile;
        pl.split_tokens = static_cast<int>(ts);
        pl.split_tail = 0;
        pl.n_splits = static_cast<int>(n_of(ts));
        pl.compact = true;
        pl.cmp_slots = static_cast<int>(std::min<long long>(slots, 0x7FFFFFFF));
        pl.cmp_step = tile;
        pl.cmp_tmax = static_cast<int>(std::min<long long>((L + tile - 1LL) / tile * tile, 0x7FFFFFC0));
    }
    if (pl.n_splits > 1) {
        const size_t bh = static_cast<size_t>(B) * H_q * std::max(qlen, 1);   // output rows
        pl.ws_ml = kWsCounterBytes;
        pl.ws_part = align_up(pl.ws_ml + bh * pl.n_splits * sizeof(float2), 256);
        pl.ws_bytes = align_up(pl.ws_part + bh * pl.n_splits * d * sizeof(float), 256);
        if (pl.compact) {
            pl.ws_nsp = pl.ws_bytes;
            pl.ws_bytes = align_up(pl.ws_nsp + units * sizeof(int), 256);
        }
        // The bf16 matrix-core kernel merges the splits of a unit in its last
        // split to finish when all its workgroups fit in one round: each
        // split then waits for its partial rows to be written and for its
        // count (a few microseconds), once, in place of a merge launch.  With
        // several rounds that wait would hold a workgroup slot every round.
        // (Partial offsets stay below 2^31 for its 32-bit buffer offsets.)
        pl.merge_in_kernel = pl.mfma && units <= kMergeCounters && units * pl.n_splits <= slots &&
                             pl.ws_bytes - pl.ws_part < (size_t{1} << 31);
    }
    // Balanced schedule (the matrix-core kernels, bf16 or uint8 cache, one
    // new token, library splits) for ragged paged pools, whose split plan
    // above is sized from the longest sequence and leaves many short or empty
    // splits, each paying a prologue.  One round of workgroups (more only if
    // a workgroup would take more than kBalMaxTokens tokens); the step count
    // must fit in 31 bits.
    // (Measured on the ragged paged workload: 202 -> 198 us.  Over a
    // contiguous cache with groups of 32 heads it was slower than the split
    // plan - 25 -> 39 us on the ragged MQA workload, whose per-segment
    // prologue and epilogue cost as much as a share of the stream - so
    // contiguous caches keep the split plan.)
    if (allow_bal && split_tokens == 0 && pl.mfma && qlen <= 1 && d <= 128 && B <= kBalMaxB &&
        units <= kMergeCounters) {
        const bool ragged_pool = pool_tokens > 0 && pool_tokens * H_kv * 10 < units * L * 9;
        const long long steps = units * ((L + tile - 1) / tile);      // >= the steps of any call
        if (ragged_pool && steps < (1LL << 31) - units) {
            const long long max_steps = kBalMaxTokens / tile;
            // (the bf16 kernel at head_dim 128 with one 16-head block: two
            // workgroups per CU, 64 KiB of tiles in flight per CU - 187 us on
            // the ragged paged workload, against 190 at the three the split
            // plan counts and 220 at one)
            const long long bal_slots =
                (!u8 && d == 128 && G <= 16) ? static_cast<long long>(cu_count()) * 2 : slots;
            const long long nwg = std::max(bal_slots, (steps + max_steps - 1) / max_steps);
            const size_t rows = static_cast<size_t>(nwg) * 2 * G;    // two partial slots per workgroup
            const size_t ml = kWsCounterBytes;
            const size_t part = align_up(ml + rows * sizeof(float2), 256);
            const size_t bytes = align_up(part + rows * d * sizeof(float), 256);
            if (bytes - part < (size_t{1} << 31) && nwg < (1LL << 24)) {
                pl.bal = true;
                pl.bal_wg = static_cast<int>(nwg);
                pl.ws_ml = ml;
                pl.ws_part = part;
                pl.ws_bytes = std::max(pl.ws_bytes, bytes);
            }
        }
    }
    *plan = pl;
    return true;
}

bool plan_mla(int B, int H, int d_latent, int max_seq_len, int split_tokens, MlaPlan* plan, const char** why) {
    MlaPlan pl{};
    pl.n_chunks = (H + kMlaHeads - 1) / kMlaHeads;
    const long long units = static_cast<long long>(B) * pl.n_chunks;
    const int L = std::max(max_seq_len, 1);
    long long ts;
    int tail = 0;       // tokens the last split may take beyond split_tokens
    auto n_of = [&](long long t) { return std::max(1LL, (L - tail + t - 1) / t); };
    if (split_tokens > 0) {
        if (split_tokens % kMlaTile != 0) {
            *why = "split_tokens must be a multiple of 32 for the latent-cache kernel";
            return false;
        }
        ts = split_tokens;
    } else {
        // One workgroup per compute unit (its LDS holds two 32-token stages
        // of d_latent-wide rows).  Each split writes H * d_latent float32
        // partials - a 32-head chunk at d_latent 512 writes 64 KiB, an eighth
        // of what a 256-token split reads - so splits stay at least 256
        // tokens long.
        const long long slots = cu_count();
        const long long S = std::max(1LL, slots / std::max(1LL, units));
        ts = (L + S - 1) / S;
        ts = std::max<long long>(ts, 256);
        ts = (ts + kMlaTile - 1) / kMlaTile * kMlaTile;
    }
    while ((L + ts - 1) / ts > kMaxSplits) ts += kMlaTile;
    if (ts > 0x7FFFFFFF) {
        *why = "split too long";
        return false;
    }
    pl.split_tokens = static_cast<int>(ts);
    pl.n_splits = static_cast<int>((L + ts - 1) / ts);
    const size_t rows = static_cast<size_t>(B) * H;
    // (after the merge counters every workspace starts with, which this
    // kernel leaves alone, so one buffer can serve both kinds of call)
    pl.qt = kWsCounterBytes;
    pl.ctx = pl.qt + align_up(rows * d_latent * sizeof(float), 256);
    pl.ws_ml = pl.ctx + align_up(rows * d_latent * sizeof(float), 256);
    pl.ws_part = pl.ws_ml + align_up(rows * pl.n_splits * sizeof(float2), 256);
    pl.ws_bytes = pl.ws_part + align_up(rows * pl.n_splits * d_latent * sizeof(float), 256);
    *plan = pl;
    return true;
}

}  // namespace kvc

extern "C" {

int kvc_abi_version(void) { return KVC_ABI_VERSION; }

const char* kvc_status_string(int status) {
    switch (status) {
        case KVC_OK: return "ok";
        case KVC_ERR_NULL: return "null pointer";
        case KVC_ERR_SHAPE: return "inconsistent sizes";
        case KVC_ERR_UNSUPPORTED: return "unsupported configuration";
        case KVC_ERR_WORKSPACE: return "workspace missing or too small";
        case KVC_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* kvc_last_error(void) { return g_last_error; }

kvc_status kvc_hbm_read_probe(const void* buf, size_t bytes, void* sink, int workgroups, int nontemporal,
                              void* stream) {
    if (!buf || !sink) return fail(KVC_ERR_NULL, "kvc_hbm_read_probe: a required pointer is NULL");
    if (bytes < 16 || workgroups <= 0)
        return fail(KVC_ERR_SHAPE, "kvc_hbm_read_probe: need bytes >= 16 and workgroups > 0");
    return hip_status(kvc::launch_read_probe(buf, bytes, static_cast<unsigned*>(sink), workgroups,
                                             nontemporal != 0, static_cast<hipStream_t>(stream)),
                      "kvc_hbm_read_probe launch");
}

void kvc_profile_next_decode(void* start_event, void* stop_event) {
    g_prof_start = static_cast<hipEvent_t>(start_event);
    g_prof_stop = static_cast<hipEvent_t>(stop_event);
}

}  // extern "C"

namespace {

kvc_status append_common(kvc_dtype dtype, int B, int H_q, int H_kv, int d, void* k_cache, void* v_cache,
                         int T_max, const int32_t* block_table, int block_size, int max_blocks_per_seq,
                         int num_blocks, const int32_t* positions, const void* k_new, const void* v_new,
                         void* q_inout, const float* rope_cos, const float* rope_sin, int rope_rows,
                         int rope_style, bool ring, void* stream, int qlen = 1) {
    kvc_status st = check_heads(dtype, B, H_q, H_kv, d);
    if (st != KVC_OK) return st;
    if (d % 2 != 0) return fail(KVC_ERR_SHAPE, "head_dim %d must be even for the rotation", d);
    if (rope_style != KVC_ROPE_INTERLEAVED && rope_style != KVC_ROPE_HALF)
        return fail(KVC_ERR_UNSUPPORTED, "unknown rope_style %d", rope_style);
    if (rope_rows <= 0) return fail(KVC_ERR_SHAPE, "rope_rows must be positive");
    if (B == 0) return ok();
    if (!k_cache || !v_cache || !positions || !k_new || !v_new || !rope_cos || !rope_sin)
        return fail(KVC_ERR_NULL, "kvc_append: a required pointer is NULL");
    kvc::AppendParams p{};
    p.dtype = dtype;
    p.B = B; p.H_q = H_q; p.H_kv = H_kv; p.d = d;
    p.k_cache = k_cache; p.v_cache = v_cache; p.T_max = T_max;
    p.block_table = block_table;
    p.block_size = block_size; p.max_blocks_per_seq = max_blocks_per_seq; p.num_blocks = num_blocks;
    if (block_table) {
        if (block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
            return fail(KVC_ERR_SHAPE, "paged append needs positive block_size, max_blocks_per_seq, num_blocks");
        const long long cap = static_cast<long long>(block_size) * max_blocks_per_seq;
        if (cap > 0x7FFFFFFF) return fail(KVC_ERR_SHAPE, "paged capacity exceeds 2^31 tokens");
        p.capacity = static_cast<int>(cap);
    } else {
        if (T_max <= 0) return fail(KVC_ERR_SHAPE, "T_max must be positive");
        p.capacity = ring ? 0x7FFFFFFF : T_max;    // a ring takes any position
    }
    p.ring = ring ? 1 : 0;
    p.qlen = qlen;
    p.positions = positions;
    p.k_new = k_new; p.v_new = v_new; p.q_inout = q_inout;
    p.rope_cos = rope_cos; p.rope_sin = rope_sin; p.rope_rows = rope_rows;
    p.rope_style = rope_style;
    return hip_status(kvc::launch_append(p, static_cast<hipStream_t>(stream)), "kvc_append launch");
}

}  // namespace

extern "C" {

kvc_status kvc_append(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                      void* k_cache, void* v_cache, int T_max,
                      const int32_t* block_table, int block_size, int max_blocks_per_seq,
                      int num_blocks, const int32_t* positions,
                      const void* k_new, const void* v_new, void* q_inout,
                      const float* rope_cos, const float* rope_sin, int rope_rows,
                      int rope_style, void* stream) {
    return append_common(dtype, B, H_q, H_kv, d, k_cache, v_cache, T_max, block_table, block_size,
                         max_blocks_per_seq, num_blocks, positions, k_new, v_new, q_inout, rope_cos, rope_sin,
                         rope_rows, rope_style, false, stream);
}

kvc_status kvc_append_ring(kvc_dtype dtype, int B, int H_q, int H_kv, int d, void* k_ring, void* v_ring,
                           int T_max, const int32_t* positions, const void* k_new, const void* v_new,
                           void* q_inout, const float* rope_cos, const float* rope_sin, int rope_rows,
                           int rope_style, void* stream) {
    return append_common(dtype, B, H_q, H_kv, d, k_ring, v_ring, T_max, nullptr, 0, 0, 0, positions, k_new,
                         v_new, q_inout, rope_cos, rope_sin, rope_rows, rope_style, true, stream);
}

kvc_status kvc_append_multi(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, void* k_cache, void* v_cache,
                            int T_max, const int32_t* block_table, int block_size, int max_blocks_per_seq,
                            int num_blocks, const int32_t* positions, const void* k_new, const void* v_new,
                            void* q_inout, const float* rope_cos, const float* rope_sin, int rope_rows,
                            int rope_style, void* stream) {
    if (n < 1) return fail(KVC_ERR_SHAPE, "tokens per sequence must be >= 1");
    return append_common(dtype, B, H_q, H_kv, d, k_cache, v_cache, T_max, block_table, block_size,
                         max_blocks_per_seq, num_blocks, positions, k_new, v_new, q_inout, rope_cos, rope_sin,
                         rope_rows, rope_style, false, stream, n);
}

int kvc_window_span(int max_seq_len, int window, int ring, int T_max) {
    if (max_seq_len < 0 || window < 0 || (ring && T_max <= 0)) return -1;
    if (ring) return std::min(max_seq_len, T_max);
    if (window > 0) return static_cast<int>(std::min<long long>(max_seq_len, static_cast<long long>(window) + 15));
    return max_seq_len;
}

}  // extern "C"

namespace {
// The append into an 8-bit cache of format fmt (KVC_U8, KVC_FP8_E4M3, KVC_FP8_E5M2).
kvc_status append_q8(kvc_dtype fmt, kvc_dtype dtype, int B, int H_q, int H_kv, int d, void* k_codes, float* k_sz,
                     void* v_codes, float* v_sz, int T_max, const int32_t* block_table, int block_size,
                     int max_blocks_per_seq, int num_blocks, const int32_t* positions, const void* k_new,
                     const void* v_new, void* q_inout, const float* rope_cos, const float* rope_sin, int rope_rows,
                     int rope_style, void* stream) {
    kvc_status st = check_heads(dtype, B, H_q, H_kv, d);
    if (st != KVC_OK) return st;
    if (d % 2 != 0 || d > 256) return fail(KVC_ERR_SHAPE, "head_dim %d must be even and at most 256", d);
    if (rope_style != KVC_ROPE_INTERLEAVED && rope_style != KVC_ROPE_HALF)
        return fail(KVC_ERR_UNSUPPORTED, "unknown rope_style %d", rope_style);
    if (rope_rows <= 0) return fail(KVC_ERR_SHAPE, "rope_rows must be positive");
    if (B == 0) return ok();
    if (!k_codes || !k_sz || !v_codes || !v_sz || !positions || !k_new || !v_new || !rope_cos || !rope_sin)
        return fail(KVC_ERR_NULL, "8-bit cache append: a required pointer is NULL");
    kvc::AppendParams p{};
    p.dtype = dtype;
    p.qfmt = q8_format(fmt);
    p.B = B; p.H_q = H_q; p.H_kv = H_kv; p.d = d;
    p.k_cache = k_codes; p.v_cache = v_codes; p.k_sz = k_sz; p.v_sz = v_sz; p.T_max = T_max;
    p.block_table = block_table;
    p.block_size = block_size; p.max_blocks_per_seq = max_blocks_per_seq; p.num_blocks = num_blocks;
    if (block_table) {
        if (block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
            return fail(KVC_ERR_SHAPE, "paged append needs positive block_size, max_blocks_per_seq, num_blocks");
        const long long cap = static_cast<long long>(block_size) * max_blocks_per_seq;
        if (cap > 0x7FFFFFFF) return fail(KVC_ERR_SHAPE, "paged capacity exceeds 2^31 tokens");
        p.capacity = static_cast<int>(cap);
    } else {
        if (T_max <= 0) return fail(KVC_ERR_SHAPE, "T_max must be positive");
        p.capacity = T_max;
    }
    p.positions = positions;
    p.k_new = k_new; p.v_new = v_new; p.q_inout = q_inout;
    p.rope_cos = rope_cos; p.rope_sin = rope_sin; p.rope_rows = rope_rows;
    p.rope_style = rope_style;
    return hip_status(kvc::launch_append_u8(p, static_cast<hipStream_t>(stream)), "8-bit cache append launch");
}

kvc_status check_fp8(kvc_dtype format) {
    if (format != KVC_FP8_E4M3 && format != KVC_FP8_E5M2)
        return fail(KVC_ERR_UNSUPPORTED, "format %d is not an FP8 cache format (KVC_FP8_E4M3 or KVC_FP8_E5M2)",
                    static_cast<int>(format));
    return KVC_OK;
}
}  // namespace

extern "C" {

kvc_status kvc_append_u8(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                         void* k_codes, float* k_sz, void* v_codes, float* v_sz, int T_max,
                         const int32_t* block_table, int block_size, int max_blocks_per_seq,
                         int num_blocks, const int32_t* positions,
                         const void* k_new, const void* v_new, void* q_inout,
                         const float* rope_cos, const float* rope_sin, int rope_rows,
                         int rope_style, void* stream) {
    return append_q8(KVC_U8, dtype, B, H_q, H_kv, d, k_codes, k_sz, v_codes, v_sz, T_max, block_table, block_size,
                     max_blocks_per_seq, num_blocks, positions, k_new, v_new, q_inout, rope_cos, rope_sin, rope_rows,
                     rope_style, stream);
}

kvc_status kvc_append_fp8(kvc_dtype format, kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                          void* k_codes, float* k_sz, void* v_codes, float* v_sz, int T_max,
                          const int32_t* block_table, int block_size, int max_blocks_per_seq,
                          int num_blocks, const int32_t* positions,
                          const void* k_new, const void* v_new, void* q_inout,
                          const float* rope_cos, const float* rope_sin, int rope_rows,
                          int rope_style, void* stream) {
    const kvc_status f = check_fp8(format);
    if (f != KVC_OK) return f;
    return append_q8(format, dtype, B, H_q, H_kv, d, k_codes, k_sz, v_codes, v_sz, T_max, block_table, block_size,
                     max_blocks_per_seq, num_blocks, positions, k_new, v_new, q_inout, rope_cos, rope_sin, rope_rows,
                     rope_style, stream);
}

size_t kvc_workspace_zeroed_bytes(void) { return kvc::kWsCounterBytes; }

size_t kvc_decode_workspace_bytes(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                                  int max_seq_len, long long pool_tokens, int split_tokens) {
    if (check_heads(is_q8(dtype) ? KVC_BF16 : dtype, B, H_q, H_kv, d) != KVC_OK || max_seq_len < 0 || split_tokens < 0 ||
        pool_tokens < 0) {
        fail(KVC_ERR_SHAPE, "invalid sizes for the decode workspace");
        return static_cast<size_t>(-1);
    }
    kvc::DecodePlan pl;
    const char* why = nullptr;
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return static_cast<size_t>(-1);
    }
    ok();
    return pl.ws_bytes;
}

int kvc_decode_split_tokens(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                            long long pool_tokens, int split_tokens) {
    if (check_heads(is_q8(dtype) ? KVC_BF16 : dtype, B, H_q, H_kv, d) != KVC_OK || max_seq_len < 0 || split_tokens < 0 ||
        pool_tokens < 0)
        return -1;
    kvc::DecodePlan pl;
    const char* why = nullptr;
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return -1;
    }
    return pl.split_tokens;
}

int kvc_decode_merge_launch(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                            long long pool_tokens, int split_tokens) {
    if (check_heads(is_q8(dtype) ? KVC_BF16 : dtype, B, H_q, H_kv, d) != KVC_OK || max_seq_len < 0 || split_tokens < 0 ||
        pool_tokens < 0)
        return -1;
    kvc::DecodePlan pl;
    const char* why = nullptr;
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return -1;
    }
    return pl.n_splits > 1 && !pl.merge_in_kernel && !pl.bal ? 1 : 0;
}

int kvc_decode_balanced(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                        long long pool_tokens, int split_tokens) {
    if (check_heads(is_q8(dtype) ? KVC_BF16 : dtype, B, H_q, H_kv, d) != KVC_OK || max_seq_len < 0 ||
        split_tokens < 0 || pool_tokens < 0)
        return -1;
    kvc::DecodePlan pl;
    const char* why = nullptr;
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return -1;
    }
    return pl.bal ? 1 : 0;
}

int kvc_decode_compact(kvc_dtype dtype, int B, int H_q, int H_kv, int d, int max_seq_len,
                       long long pool_tokens, int split_tokens) {
    if (check_heads(is_q8(dtype) ? KVC_BF16 : dtype, B, H_q, H_kv, d) != KVC_OK || max_seq_len < 0 ||
        split_tokens < 0 || pool_tokens < 0)
        return -1;
    kvc::DecodePlan pl;
    const char* why = nullptr;
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, max_seq_len, pool_tokens, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return -1;
    }
    return pl.compact ? 1 : 0;
}

namespace {
// plan of a multi-token call (sizes as kvc_decode_attn_multi's); false if invalid
bool plan_multi(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, int max_seq_len, int window,
                long long pool_tokens, int split_tokens, kvc::DecodePlan* pl) {
    if (n < 1 || window < 0 || check_heads(dtype, B, H_q, H_kv, d) != KVC_OK || max_seq_len < 0 ||
        split_tokens < 0 || pool_tokens < 0) {
        fail(KVC_ERR_SHAPE, "invalid sizes for a multi-token decode");
        return false;
    }
    const char* why = nullptr;
    const int span = kvc_window_span(max_seq_len, window > 0 ? window + n - 1 : 0, 0, 0);
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, span, pool_tokens, split_tokens, pl, &why, n, false)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return false;
    }
    return true;
}
}  // namespace

size_t kvc_decode_multi_workspace_bytes(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, int max_seq_len,
                                        int window, long long pool_tokens, int split_tokens) {
    kvc::DecodePlan pl;
    if (!plan_multi(dtype, B, n, H_q, H_kv, d, max_seq_len, window, pool_tokens, split_tokens, &pl))
        return static_cast<size_t>(-1);
    ok();
    return pl.ws_bytes;
}

int kvc_decode_multi_split_tokens(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, int max_seq_len,
                                  int window, long long pool_tokens, int split_tokens) {
    kvc::DecodePlan pl;
    if (!plan_multi(dtype, B, n, H_q, H_kv, d, max_seq_len, window, pool_tokens, split_tokens, &pl)) return -1;
    return pl.split_tokens;
}

}  // extern "C"

namespace {

// The append half of kvc_decode_step (NULL for a plain decode call).
struct StepArgs {
    const int32_t* positions;
    const void* k_new;
    const void* v_new;
    void* q_rot_out;
    const float* rope_cos;
    const float* rope_sin;
    int rope_rows;
    int rope_style;
};

// dtype KVC_U8: k / v are uint8 codes with pairs k_sz / v_sz (q and out bf16).
kvc_status decode_common(kvc_dtype dtype, int B, int H_q, int H_kv, int d, const void* q,
                         const void* k, const void* v, int T_max, int num_blocks, int block_size,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                         int split_tokens, void* workspace, size_t workspace_bytes, void* stream,
                         const StepArgs* step, const float* k_sz = nullptr, const float* v_sz = nullptr,
                         int window = 0, int ring = 0, int qlen = 0) {
    // qlen: 0 for the single-token entry points; n >= 1 for kvc_decode_attn_multi
    // (whose matrix-core launches use the multi-token rows even for n = 1)
    const bool multi = qlen > 0;
    qlen = multi ? qlen : 1;
    const hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;   // one-shot, cleared by every call
    g_prof_start = g_prof_stop = nullptr;
    const bool u8 = is_q8(dtype);
    kvc_status st = check_heads(u8 ? KVC_BF16 : dtype, B, H_q, H_kv, d);
    if (st != KVC_OK) return st;
    if (u8 && B > 0 && (!k_sz || !v_sz)) return fail(KVC_ERR_NULL, "quantized decode: k_sz or v_sz is NULL");
    const bool paged = block_table != nullptr;
    if (max_seq_len < 0) return fail(KVC_ERR_SHAPE, "max_seq_len must be >= 0");
    if (split_tokens < 0) return fail(KVC_ERR_SHAPE, "split_tokens must be >= 0");
    if (window < 0) return fail(KVC_ERR_SHAPE, "window must be >= 0");
    if (ring && paged) return fail(KVC_ERR_UNSUPPORTED, "a ring cache is contiguous (no block table)");
    if (ring && window != 0 && window != T_max)
        return fail(KVC_ERR_SHAPE, "a ring of T_max = %d slots attends all of them: window must be 0 or %d", T_max,
                    T_max);
    if (u8 && (window || ring)) return fail(KVC_ERR_UNSUPPORTED, "no sliding window for the quantized cache");
    if (multi && (u8 || ring || step))
        return fail(KVC_ERR_UNSUPPORTED, "several new tokens: bf16 over a full cache, append first");
    if (paged) {
        if (block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
            return fail(KVC_ERR_SHAPE, "paged decode needs positive block_size, max_blocks_per_seq, num_blocks");
        if (static_cast<long long>(max_seq_len) > static_cast<long long>(block_size) * max_blocks_per_seq)
            return fail(KVC_ERR_SHAPE, "max_seq_len %d exceeds the block table's %lld tokens", max_seq_len,
                        static_cast<long long>(block_size) * max_blocks_per_seq);
    } else if (ring) {
        if (T_max <= 0) return fail(KVC_ERR_SHAPE, "T_max must be positive");
    } else if (max_seq_len > T_max) {
        return fail(KVC_ERR_SHAPE, "max_seq_len %d exceeds the cache capacity T_max %d", max_seq_len, T_max);
    }
    if (step) {
        if (d % 2 != 0) return fail(KVC_ERR_SHAPE, "head_dim %d must be even for the rotation", d);
        if (step->rope_style != KVC_ROPE_INTERLEAVED && step->rope_style != KVC_ROPE_HALF)
            return fail(KVC_ERR_UNSUPPORTED, "unknown rope_style %d", step->rope_style);
        if (step->rope_rows <= 0) return fail(KVC_ERR_SHAPE, "rope_rows must be positive");
    }
    if (B == 0) return ok();
    if (!q || !k || !v || !out || (!step && !seq_lens))
        return fail(KVC_ERR_NULL, "decode: a required pointer is NULL");
    if (step && (!step->positions || !step->k_new || !step->v_new || !step->q_rot_out || !step->rope_cos ||
                 !step->rope_sin))
        return fail(KVC_ERR_NULL, "kvc_decode_step: a required pointer is NULL");
    kvc::DecodePlan pl;
    const char* why = nullptr;
    const long long pool_tokens = paged ? static_cast<long long>(num_blocks) * block_size : 0;
    // splits cover the attended span of a sequence (a window's tokens, or the
    // ring's slots), which kvc_window_span gives
    // (several new tokens: the first one's window starts qlen - 1 tokens earlier)
    const int span = kvc_window_span(max_seq_len, window > 0 ? window + qlen - 1 : 0, ring, T_max);
    if (!kvc::plan_decode(dtype, B, H_q, H_kv, d, span, pool_tokens, split_tokens, &pl, &why, qlen))
        return fail(KVC_ERR_UNSUPPORTED, "%s", why);
    // the balanced schedule serves one new token over a full paged cache of
    // blocks of a multiple of 16 tokens; other calls take the split plan,
    // whose workspace the balanced plan's size covers
    if (((pl.bal && (multi || window != 0 || ring || !paged || block_size % 16 != 0)) || (pl.compact && multi)) &&
        !kvc::plan_decode(dtype, B, H_q, H_kv, d, span, pool_tokens, split_tokens, &pl, &why, qlen, false))
        return fail(KVC_ERR_UNSUPPORTED, "%s", why);
    if (u8 && paged) {
        // 32-token tiles of 16-row groups, each inside one block, found in a
        // staged slice of at most kTblMax table entries
        if (pl.split_tokens % 16 != 0)
            return fail(KVC_ERR_UNSUPPORTED, "the quantized paged kernel needs split_tokens a multiple of 16");
        if (std::min(pl.split_tokens, std::max(max_seq_len, 1)) / block_size + 2 > kvc::kTblMax)
            return fail(KVC_ERR_UNSUPPORTED, "a split of the quantized paged kernel spans more than %d blocks",
                        kvc::kTblMax - 2);
    }
    if (pl.ws_bytes > 0) {
        if (!workspace) return fail(KVC_ERR_WORKSPACE, "decode needs %zu bytes of workspace, got NULL", pl.ws_bytes);
        if (workspace_bytes < pl.ws_bytes)
            return fail(KVC_ERR_WORKSPACE, "decode needs %zu bytes of workspace, got %zu", pl.ws_bytes, workspace_bytes);
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return fail(KVC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    const long long n_wg = pl.bal ? pl.bal_wg : static_cast<long long>(B) * H_kv * pl.n_chunks * pl.n_splits;
    if (n_wg > 0x7FFFFFF0LL) return fail(KVC_ERR_SHAPE, "too many workgroups");

    kvc::DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.seq_lens = seq_lens;
    p.block_table = block_table;
    char* ws = static_cast<char*>(workspace);
    p.ws_part = pl.ws_bytes ? reinterpret_cast<float*>(ws + pl.ws_part) : nullptr;
    p.ws_ml = pl.ws_bytes ? reinterpret_cast<float2*>(ws + pl.ws_ml) : nullptr;
    // the matrix-core kernels merge the splits themselves when the plan says
    // so: the last split of each unit to finish (counted in the workspace's
    // first bytes) does it
    const bool merge_in_kernel = pl.merge_in_kernel || pl.bal;
    p.merge_cnt = merge_in_kernel ? reinterpret_cast<unsigned*>(ws) : nullptr;
    p.bal = pl.bal ? 1 : 0;
    p.compact = pl.compact ? 1 : 0;
    p.ws_nsp = pl.compact && pl.ws_bytes ? reinterpret_cast<int*>(ws + pl.ws_nsp) : nullptr;
    p.cmp_slots = pl.cmp_slots;
    p.cmp_step = pl.cmp_step;
    p.cmp_tmax = pl.cmp_tmax;
    p.B = B; p.H_q = H_q; p.H_kv = H_kv; p.G = H_q / H_kv; p.n_chunks = pl.n_chunks;
    p.T_max = T_max; p.block_size = block_size; p.max_blocks_per_seq = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.max_seq_len = max_seq_len; p.split_tokens = pl.split_tokens; p.n_splits = pl.n_splits;
    p.split_tail = pl.split_tail;
    p.window = ring ? 0 : window;
    p.ring = ring ? 1 : 0;
    p.align = paged ? 16 : 1;
    p.qlen = qlen;
    p.n_wg = static_cast<int>(n_wg);
    p.n_wg_pad = static_cast<int>((n_wg + 7) / 8 * 8);
    const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(d));
    p.scale_log2 = sc * 1.4426950408889634f;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    kvc::KernelTiming tm;
    tm.start = ev0;
    tm.stop = ev1;
    hipError_t e = hipSuccess;
    // the append runs inside the matrix-core kernel, except for a ring (the new
    // token's slot is not the last attended row there)
    const bool fused = step != nullptr && pl.mfma && !ring;
    // ... and inside the vector kernel for a contiguous cache (one new token)
    const bool valu_step = step != nullptr && !pl.mfma && !ring && !paged && qlen <= 1;
    if (step) {
        p.positions = step->positions;
        p.k_new = step->k_new;
        p.v_new = step->v_new;
        p.q_raw = q;
        p.q_rot_out = step->q_rot_out;
        p.rope_cos = step->rope_cos;
        p.rope_sin = step->rope_sin;
        p.rope_rows = step->rope_rows;
        p.rope_style = step->rope_style;
        p.capacity = paged ? block_size * max_blocks_per_seq : (ring ? 0x7FFFFFFF : T_max);
        p.seq_lens = nullptr;
        p.valu_step = valu_step ? 1 : 0;
        if (!fused && !valu_step) {
            // no fused kernel for this shape (or a ring cache): the append
            // (which also rotates q into q_rot_out), then the attention
            kvc::AppendParams ap{};
            ap.dtype = dtype;
            ap.B = B; ap.H_q = H_q; ap.H_kv = H_kv; ap.d = d;
            ap.k_cache = const_cast<void*>(k); ap.v_cache = const_cast<void*>(v); ap.T_max = T_max;
            ap.block_table = block_table; ap.block_size = block_size;
            ap.max_blocks_per_seq = max_blocks_per_seq; ap.num_blocks = num_blocks;
            ap.capacity = p.capacity;
            ap.positions = step->positions;
            ap.k_new = step->k_new; ap.v_new = step->v_new; ap.q_inout = step->q_rot_out; ap.q_in = q;
            ap.rope_cos = step->rope_cos; ap.rope_sin = step->rope_sin;
            ap.rope_rows = step->rope_rows; ap.rope_style = step->rope_style;
            ap.ring = p.ring;
            e = kvc::launch_append(ap, hs);
            if (e != hipSuccess) return hip_status(e, "kvc_decode_step append launch");
            p.q = step->q_rot_out;
        }
    }
    if (u8)
        e = kvc::launch_decode_u8(d, p.G, paged, fused, q8_format(dtype), p, const_cast<float*>(k_sz),
                                  const_cast<float*>(v_sz), hs, tm);
    else e = pl.mfma ? kvc::launch_decode_mfma(d, qlen > 1 ? pl.heads_per_wg : p.G, paged, fused, multi, p, hs, tm)
                     : kvc::launch_decode_split(dtype, d, pl.heads_per_wg, paged, p, hs, tm);
    if (e != hipSuccess) return hip_status(e, "decode split launch");
    if (pl.n_splits > 1 && !merge_in_kernel) {
        e = kvc::launch_decode_merge(u8 ? KVC_BF16 : dtype, d, p, hs);
        if (e != hipSuccess) return hip_status(e, "decode merge launch");
    }
    return ok();
}

}  // namespace

extern "C" {

kvc_status kvc_decode_attn(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                           const void* q, const void* k_cache, const void* v_cache, int T_max,
                           const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                           int split_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, T_max, 0, 0, nullptr, 0, seq_lens,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, nullptr);
}

kvc_status kvc_decode_attn_paged(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 int num_blocks, int block_size, const int32_t* block_table,
                                 int max_blocks_per_seq, const int32_t* seq_lens,
                                 int max_seq_len, float scale, void* out, int split_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_table) return fail(KVC_ERR_NULL, "kvc_decode_attn_paged: block_table is NULL");
    return decode_common(dtype, B, H_q, H_kv, d, q, k_pool, v_pool, 0, num_blocks, block_size, block_table,
                         max_blocks_per_seq, seq_lens, max_seq_len, scale, out, split_tokens, workspace,
                         workspace_bytes, stream, nullptr);
}

kvc_status kvc_decode_step(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                           const void* q, void* q_rot_out, void* k_cache, void* v_cache, int T_max,
                           const int32_t* block_table, int block_size, int max_blocks_per_seq,
                           int num_blocks, const int32_t* positions, const void* k_new,
                           const void* v_new, const float* rope_cos, const float* rope_sin,
                           int rope_rows, int rope_style, int max_seq_len, float scale, void* out,
                           int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    StepArgs st{positions, k_new, v_new, q_rot_out, rope_cos, rope_sin, rope_rows, rope_style};
    if (block_table)
        return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, 0, num_blocks, block_size,
                             block_table, max_blocks_per_seq, nullptr, max_seq_len, scale, out, split_tokens,
                             workspace, workspace_bytes, stream, &st);
    return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, T_max, 0, 0, nullptr, 0, nullptr,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, &st);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// kvc_decode_step_noalloc: kvc_decode_step with its workspace in a fixed
// array of device memory that the library owns, for callers that cannot
// allocate.  Each device the library runs on holds its own copy of `scratch`
// until the process ends; its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// handed to kernels - the array's name in host code is not a device address.
// The split partials it holds are written before they are read in every
// call, so nothing needs clearing; every call on a device shares the array,
// so calls that overlap on one device race.
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // device address of `scratch` per device (nullptr: not looked up)

kvc_status scratch_address(void** addr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "kvc_decode_step_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_step_noalloc: device index %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "kvc_decode_step_noalloc: hipGetSymbolAddress(scratch)");
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0)
            return fail(KVC_ERR_HIP, "kvc_decode_step_noalloc: scratch address %p unusable", p);
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return KVC_OK;
}

}  // namespace

extern "C" {

size_t kvc_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

kvc_status kvc_decode_step_noalloc(kvc_dtype dtype, int B, int H_q, int H_kv, int d,
                                   const void* q, void* q_rot_out, void* k_cache, void* v_cache, int T_max,
                                   const int32_t* block_table, int block_size, int max_blocks_per_seq,
                                   int num_blocks, const int32_t* positions, const void* k_new,
                                   const void* v_new, const float* rope_cos, const float* rope_sin,
                                   int rope_rows, int rope_style, int max_seq_len, float scale, void* out,
                                   int split_tokens, void* stream) {
    // the plan's workspace, checked against the fixed array before any HIP
    // call (invalid sizes fall through to kvc_decode_step, which names them)
    const long long pool_tokens =
        block_table ? static_cast<long long>(num_blocks) * std::max(block_size, 0) : 0;
    const size_t need = (B > 0 && max_seq_len >= 0 && pool_tokens >= 0)
                            ? kvc_decode_workspace_bytes(dtype, B, H_q, H_kv, d, max_seq_len, pool_tokens,
                                                         split_tokens)
                            : 0;
    if (need != static_cast<size_t>(-1) && need > kScratchBytes)
        return fail(KVC_ERR_WORKSPACE,
                    "kvc_decode_step_noalloc: this call needs %zu bytes of split partials, more than the %zu bytes "
                    "of the library's fixed scratch (use kvc_decode_step with a workspace, or longer splits)",
                    need, kScratchBytes);
    if (B > 0 && (!q || !q_rot_out || !k_cache || !v_cache || !out || !positions || !k_new || !v_new || !rope_cos ||
                  !rope_sin))
        return fail(KVC_ERR_NULL, "kvc_decode_step_noalloc: a required pointer is NULL");
    void* ws = nullptr;
    if (B > 0 && need != static_cast<size_t>(-1)) {   // (invalid sizes: kvc_decode_step reports them)
        const kvc_status st = scratch_address(&ws);
        if (st != KVC_OK) return st;
    }
    return kvc_decode_step(dtype, B, H_q, H_kv, d, q, q_rot_out, k_cache, v_cache, T_max, block_table, block_size,
                           max_blocks_per_seq, num_blocks, positions, k_new, v_new, rope_cos, rope_sin, rope_rows,
                           rope_style, max_seq_len, scale, out, split_tokens, ws, kScratchBytes, stream);
}

kvc_status kvc_decode_attn_window(kvc_dtype dtype, int B, int H_q, int H_kv, int d, const void* q,
                                  const void* k_cache, const void* v_cache, int T_max, const int32_t* block_table,
                                  int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* seq_lens,
                                  int max_seq_len, int window, int ring, float scale, void* out, int split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (block_table)
        return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, 0, num_blocks, block_size, block_table,
                             max_blocks_per_seq, seq_lens, max_seq_len, scale, out, split_tokens, workspace,
                             workspace_bytes, stream, nullptr, nullptr, nullptr, window, ring);
    return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, T_max, 0, 0, nullptr, 0, seq_lens,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, nullptr, nullptr,
                         nullptr, window, ring);
}

kvc_status kvc_decode_step_window(kvc_dtype dtype, int B, int H_q, int H_kv, int d, const void* q, void* q_rot_out,
                                  void* k_cache, void* v_cache, int T_max, const int32_t* block_table,
                                  int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* positions,
                                  const void* k_new, const void* v_new, const float* rope_cos,
                                  const float* rope_sin, int rope_rows, int rope_style, int max_seq_len,
                                  int window, int ring, float scale, void* out, int split_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    StepArgs st{positions, k_new, v_new, q_rot_out, rope_cos, rope_sin, rope_rows, rope_style};
    if (block_table)
        return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, 0, num_blocks, block_size,
                             block_table, max_blocks_per_seq, nullptr, max_seq_len, scale, out, split_tokens,
                             workspace, workspace_bytes, stream, &st, nullptr, nullptr, window, ring);
    return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, T_max, 0, 0, nullptr, 0, nullptr,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, &st, nullptr,
                         nullptr, window, ring);
}

kvc_status kvc_decode_attn_multi(kvc_dtype dtype, int B, int n, int H_q, int H_kv, int d, const void* q,
                                 const void* k_cache, const void* v_cache, int T_max, const int32_t* block_table,
                                 int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* seq_lens,
                                 int max_seq_len, int window, float scale, void* out, int split_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 1) return fail(KVC_ERR_SHAPE, "tokens per sequence must be >= 1");
    if (block_table)
        return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, 0, num_blocks, block_size, block_table,
                             max_blocks_per_seq, seq_lens, max_seq_len, scale, out, split_tokens, workspace,
                             workspace_bytes, stream, nullptr, nullptr, nullptr, window, 0, n);
    return decode_common(dtype, B, H_q, H_kv, d, q, k_cache, v_cache, T_max, 0, 0, nullptr, 0, seq_lens,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, nullptr, nullptr,
                         nullptr, window, 0, n);
}

kvc_status kvc_decode_attn_u8(int B, int H_q, int H_kv, int d, const void* q, const void* k_codes,
                              const float* k_sz, const void* v_codes, const float* v_sz, int T_max,
                              const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                              int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_common(KVC_U8, B, H_q, H_kv, d, q, k_codes, v_codes, T_max, 0, 0, nullptr, 0, seq_lens,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, nullptr,
                         k_sz, v_sz);
}

kvc_status kvc_decode_attn_paged_u8(int B, int H_q, int H_kv, int d, const void* q, const void* k_codes,
                                    const float* k_sz, const void* v_codes, const float* v_sz, int num_blocks,
                                    int block_size, const int32_t* block_table, int max_blocks_per_seq,
                                    const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                                    int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_table) return fail(KVC_ERR_NULL, "kvc_decode_attn_paged_u8: block_table is NULL");
    if (block_size % 16 != 0)
        return fail(KVC_ERR_UNSUPPORTED, "the quantized paged kernel needs block_size a multiple of 16");
    return decode_common(KVC_U8, B, H_q, H_kv, d, q, k_codes, v_codes, 0, num_blocks, block_size, block_table,
                         max_blocks_per_seq, seq_lens, max_seq_len, scale, out, split_tokens, workspace,
                         workspace_bytes, stream, nullptr, k_sz, v_sz);
}

kvc_status kvc_decode_step_u8(int B, int H_q, int H_kv, int d, const void* q, void* q_rot_out, void* k_codes,
                              float* k_sz, void* v_codes, float* v_sz, int T_max, const int32_t* block_table,
                              int block_size, int max_blocks_per_seq, int num_blocks, const int32_t* positions,
                              const void* k_new, const void* v_new, const float* rope_cos, const float* rope_sin,
                              int rope_rows, int rope_style, int max_seq_len, float scale, void* out,
                              int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    StepArgs st{positions, k_new, v_new, q_rot_out, rope_cos, rope_sin, rope_rows, rope_style};
    if (block_table) {
        if (block_size % 16 != 0)
            return fail(KVC_ERR_UNSUPPORTED, "the quantized paged kernel needs block_size a multiple of 16");
        return decode_common(KVC_U8, B, H_q, H_kv, d, q, k_codes, v_codes, 0, num_blocks, block_size, block_table,
                             max_blocks_per_seq, nullptr, max_seq_len, scale, out, split_tokens, workspace,
                             workspace_bytes, stream, &st, k_sz, v_sz);
    }
    return decode_common(KVC_U8, B, H_q, H_kv, d, q, k_codes, v_codes, T_max, 0, 0, nullptr, 0, nullptr,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, &st, k_sz, v_sz);
}

kvc_status kvc_decode_attn_fp8(kvc_dtype format, int B, int H_q, int H_kv, int d, const void* q,
                               const void* k_codes, const float* k_sz, const void* v_codes, const float* v_sz,
                               int T_max, const int32_t* seq_lens, int max_seq_len, float scale, void* out,
                               int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    const kvc_status f = check_fp8(format);
    if (f != KVC_OK) return f;
    return decode_common(format, B, H_q, H_kv, d, q, k_codes, v_codes, T_max, 0, 0, nullptr, 0, seq_lens,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, nullptr,
                         k_sz, v_sz);
}

kvc_status kvc_decode_attn_paged_fp8(kvc_dtype format, int B, int H_q, int H_kv, int d, const void* q,
                                     const void* k_codes, const float* k_sz, const void* v_codes,
                                     const float* v_sz, int num_blocks, int block_size, const int32_t* block_table,
                                     int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, float scale,
                                     void* out, int split_tokens, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    const kvc_status f = check_fp8(format);
    if (f != KVC_OK) return f;
    if (!block_table) return fail(KVC_ERR_NULL, "kvc_decode_attn_paged_fp8: block_table is NULL");
    if (block_size % 16 != 0)
        return fail(KVC_ERR_UNSUPPORTED, "the 8-bit paged kernel needs block_size a multiple of 16");
    return decode_common(format, B, H_q, H_kv, d, q, k_codes, v_codes, 0, num_blocks, block_size, block_table,
                         max_blocks_per_seq, seq_lens, max_seq_len, scale, out, split_tokens, workspace,
                         workspace_bytes, stream, nullptr, k_sz, v_sz);
}

kvc_status kvc_decode_step_fp8(kvc_dtype format, int B, int H_q, int H_kv, int d, const void* q, void* q_rot_out,
                               void* k_codes, float* k_sz, void* v_codes, float* v_sz, int T_max,
                               const int32_t* block_table, int block_size, int max_blocks_per_seq, int num_blocks,
                               const int32_t* positions, const void* k_new, const void* v_new,
                               const float* rope_cos, const float* rope_sin, int rope_rows, int rope_style,
                               int max_seq_len, float scale, void* out, int split_tokens, void* workspace,
                               size_t workspace_bytes, void* stream) {
    const kvc_status f = check_fp8(format);
    if (f != KVC_OK) return f;
    StepArgs st{positions, k_new, v_new, q_rot_out, rope_cos, rope_sin, rope_rows, rope_style};
    if (block_table) {
        if (block_size % 16 != 0)
            return fail(KVC_ERR_UNSUPPORTED, "the 8-bit paged kernel needs block_size a multiple of 16");
        return decode_common(format, B, H_q, H_kv, d, q, k_codes, v_codes, 0, num_blocks, block_size, block_table,
                             max_blocks_per_seq, nullptr, max_seq_len, scale, out, split_tokens, workspace,
                             workspace_bytes, stream, &st, k_sz, v_sz);
    }
    return decode_common(format, B, H_q, H_kv, d, q, k_codes, v_codes, T_max, 0, 0, nullptr, 0, nullptr,
                         max_seq_len, scale, out, split_tokens, workspace, workspace_bytes, stream, &st, k_sz, v_sz);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Latent cache (multi-head latent attention)
// ---------------------------------------------------------------------------

namespace {

kvc_status check_mla_sizes(int B, int H, int d_latent, int rope_dim, int max_seq_len, int split_tokens) {
    if (B < 0 || H <= 0 || rope_dim < 0 || max_seq_len < 0 || split_tokens < 0)
        return fail(KVC_ERR_SHAPE, "latent cache: invalid sizes (B=%d H=%d rope_dim=%d max_seq_len=%d)", B, H,
                    rope_dim, max_seq_len);
    if (d_latent != 128 && d_latent != 256 && d_latent != 512)
        return fail(KVC_ERR_UNSUPPORTED, "latent cache: d_latent %d must be 128, 256 or 512", d_latent);
    if ((d_latent + rope_dim) % 8 != 0)
        return fail(KVC_ERR_SHAPE, "latent cache: d_latent + rope_dim = %d must be a multiple of 8",
                    d_latent + rope_dim);
    return KVC_OK;
}

kvc_status mla_common(int B, int H, int d_k, int d_latent, int rope_dim, const void* q, void* cache, int T_max,
                      const int32_t* seq_lens, const int32_t* positions, const void* c_new, const void* r_new,
                      int max_seq_len, const void* w_uk, const void* w_uv, const void* b_uv, float scale,
                      float* out, int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    const hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;   // one-shot, cleared by every call
    g_prof_start = g_prof_stop = nullptr;
    kvc_status st = check_mla_sizes(B, H, d_latent, rope_dim, max_seq_len, split_tokens);
    if (st != KVC_OK) return st;
    if (d_k <= 0 || d_k % 32 != 0 || d_k > 512)
        return fail(KVC_ERR_UNSUPPORTED, "latent cache: d_k %d must be a positive multiple of 32, at most 512", d_k);
    if (T_max <= 0) return fail(KVC_ERR_SHAPE, "T_max must be positive");
    if (max_seq_len > T_max)
        return fail(KVC_ERR_SHAPE, "max_seq_len %d exceeds the cache capacity T_max %d", max_seq_len, T_max);
    const int row = d_latent + rope_dim;
    if (static_cast<long long>(T_max) * row * 2 + 2LL * kvc::kMlaTile * row * 2 >= 0x7FFFFFFFLL)
        return fail(KVC_ERR_SHAPE, "latent cache: one sequence's rows exceed 2 GiB");
    if (B == 0) return ok();
    if (!q || !cache || !w_uk || !w_uv || !out || (!positions && !seq_lens))
        return fail(KVC_ERR_NULL, "latent-cache decode: a required pointer is NULL");
    if (positions && (!c_new || (rope_dim > 0 && !r_new)))
        return fail(KVC_ERR_NULL, "kvc_decode_step_mla: c_kv_new or k_rope_new is NULL");
    kvc::MlaPlan pl;
    const char* why = nullptr;
    if (!kvc::plan_mla(B, H, d_latent, max_seq_len, split_tokens, &pl, &why))
        return fail(KVC_ERR_UNSUPPORTED, "%s", why);
    if (!workspace) return fail(KVC_ERR_WORKSPACE, "latent-cache decode needs %zu bytes of workspace, got NULL",
                                pl.ws_bytes);
    if (workspace_bytes < pl.ws_bytes)
        return fail(KVC_ERR_WORKSPACE, "latent-cache decode needs %zu bytes of workspace, got %zu", pl.ws_bytes,
                    workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(KVC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const long long n_wg = static_cast<long long>(B) * pl.n_chunks * pl.n_splits;
    if (n_wg > 0x7FFFFFF0LL) return fail(KVC_ERR_SHAPE, "too many workgroups");
    kvc::MlaParams p{};
    p.q = q; p.cache = cache; p.seq_lens = seq_lens; p.positions = positions;
    p.c_new = positions ? c_new : nullptr;
    p.r_new = r_new;
    p.w_uk = w_uk; p.w_uv = w_uv; p.b_uv = b_uv; p.out = out;
    char* ws = static_cast<char*>(workspace);
    p.qt = reinterpret_cast<float*>(ws + pl.qt);
    p.ctx = reinterpret_cast<float*>(ws + pl.ctx);
    p.ws_ml = reinterpret_cast<float2*>(ws + pl.ws_ml);
    p.ws_part = reinterpret_cast<float*>(ws + pl.ws_part);
    p.B = B; p.H = H; p.d_k = d_k; p.d_latent = d_latent; p.rope_dim = rope_dim; p.row = row;
    p.T_max = T_max; p.max_seq_len = max_seq_len;
    p.split_tokens = pl.split_tokens; p.n_splits = pl.n_splits; p.n_chunks = pl.n_chunks;
    p.n_wg = static_cast<int>(n_wg);
    const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(d_k));
    p.scale_log2 = sc * 1.4426950408889634f;
    kvc::KernelTiming tm;
    tm.start = ev0;
    tm.stop = ev1;
    return hip_status(kvc::launch_mla(p, static_cast<hipStream_t>(stream), tm), "latent-cache decode launch");
}

}  // namespace

extern "C" {

kvc_status kvc_append_mla(kvc_dtype dtype, int B, int d_latent, int rope_dim, void* cache, int T_max,
                          const int32_t* positions, const void* c_kv_new, const void* k_rope_new, void* stream) {
    if (dtype != KVC_BF16 && dtype != KVC_F32) return fail(KVC_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (B < 0 || d_latent <= 0 || rope_dim < 0 || T_max <= 0)
        return fail(KVC_ERR_SHAPE, "kvc_append_mla: invalid sizes (B=%d d_latent=%d rope_dim=%d T_max=%d)", B,
                    d_latent, rope_dim, T_max);
    if ((d_latent + rope_dim) % 8 != 0)
        return fail(KVC_ERR_SHAPE, "kvc_append_mla: d_latent + rope_dim = %d must be a multiple of 8",
                    d_latent + rope_dim);
    if (B == 0) return ok();
    if (!cache || !positions || !c_kv_new || (rope_dim > 0 && !k_rope_new))
        return fail(KVC_ERR_NULL, "kvc_append_mla: a required pointer is NULL");
    return hip_status(kvc::launch_append_mla(static_cast<int>(elem_bytes(dtype)), B, d_latent, rope_dim, cache,
                                             T_max, positions, c_kv_new, k_rope_new,
                                             static_cast<hipStream_t>(stream)),
                      "kvc_append_mla launch");
}

size_t kvc_decode_mla_workspace_bytes(int B, int H, int d_latent, int max_seq_len, int split_tokens) {
    if (check_mla_sizes(B, H, d_latent, 0, max_seq_len, split_tokens) != KVC_OK) return static_cast<size_t>(-1);
    kvc::MlaPlan pl;
    const char* why = nullptr;
    if (!kvc::plan_mla(B, H, d_latent, max_seq_len, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return static_cast<size_t>(-1);
    }
    ok();
    return pl.ws_bytes;
}

int kvc_decode_mla_split_tokens(int B, int H, int d_latent, int max_seq_len, int split_tokens) {
    if (check_mla_sizes(B, H, d_latent, 0, max_seq_len, split_tokens) != KVC_OK) return -1;
    kvc::MlaPlan pl;
    const char* why = nullptr;
    if (!kvc::plan_mla(B, H, d_latent, max_seq_len, split_tokens, &pl, &why)) {
        fail(KVC_ERR_UNSUPPORTED, "%s", why);
        return -1;
    }
    return pl.split_tokens;
}

kvc_status kvc_decode_attn_mla(int B, int H, int d_k, int d_latent, int rope_dim, const void* q,
                               const void* cache, int T_max, const int32_t* seq_lens, int max_seq_len,
                               const void* w_uk, const void* w_uv, const void* b_uv, float scale, float* out,
                               int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    if (B > 0 && !seq_lens) return fail(KVC_ERR_NULL, "kvc_decode_attn_mla: seq_lens is NULL");
    return mla_common(B, H, d_k, d_latent, rope_dim, q, const_cast<void*>(cache), T_max, seq_lens, nullptr,
                      nullptr, nullptr, max_seq_len, w_uk, w_uv, b_uv, scale, out, split_tokens, workspace,
                      workspace_bytes, stream);
}

kvc_status kvc_decode_step_mla(int B, int H, int d_k, int d_latent, int rope_dim, const void* q, void* cache,
                               int T_max, const int32_t* positions, const void* c_kv_new,
                               const void* k_rope_new, int max_seq_len, const void* w_uk, const void* w_uv,
                               const void* b_uv, float scale, float* out, int split_tokens, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (B > 0 && !positions) return fail(KVC_ERR_NULL, "kvc_decode_step_mla: positions is NULL");
    return mla_common(B, H, d_k, d_latent, rope_dim, q, cache, T_max, nullptr, positions, c_kv_new, k_rope_new,
                      max_seq_len, w_uk, w_uv, b_uv, scale, out, split_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"
