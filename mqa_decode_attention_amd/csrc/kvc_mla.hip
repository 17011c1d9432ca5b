// kvc_mla.hip - decode attention over a latent cache (multi-head latent
// attention) on the gfx950 matrix cores.
//
// The operation is the one of the MultiHeadLatentAttention listing in "KV
// Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략"
// (youngju.dev): a token is cached as its latent c_t (d_latent values) and a
// rope part, and head h sees key W_uk,h c_t + b_uk,h and value W_uv,h c_t +
// b_uv,h.  It is computed in the absorbed form, which is exact:
//
//   q~_h   = W_uk,h^T q_h                      (mla_absorb_kernel)
//   s_h,t  = scale * q~_h . c_t                (the key bias only adds
//                                               scale * q_h . b_uk,h to every
//                                               score of head h: the softmax
//                                               removes it)
//   x_h    = sum_t softmax(s_h)_t c_t          (mla_decode_kernel, split over
//                                               tokens; mla_merge_kernel)
//   out_h  = W_uv,h x_h + b_uv,h               (mla_up_kernel; the weights sum
//                                               to 1, so the value bias comes
//                                               out once)
//
// so the cache is streamed once, d_latent values per token, and every latent
// row serves as the key and the value of all heads at once.
//
// mla_decode_kernel: one workgroup of four waves per (sequence, chunk of up
// to 32 heads, token split).  The split's rows pass through LDS in 32-token
// tiles (direct loads, NST stages).  Wave w owns latent columns
// [w * d_latent / 4, (w + 1) * d_latent / 4):
//   * scores: the wave multiplies its column slice of the tile by the same
//     slice of the absorbed queries (v_mfma_f32_16x16x32_bf16, S^T = C Q~^T,
//     16 tokens x 16 heads per product) and leaves its partial sums in LDS;
//     after a barrier every wave adds the four partials in the same order,
//     so all four hold bit-identical scores and run the same online softmax;
//   * PV: the wave accumulates its columns of X^T += C^T P^T, C^T read
//     transposed from the staged tile (ds_read_b64_tr_b16).
// The absorbed queries and the probabilities enter the products as hi + lo
// pairs of bf16 (about 16 significant bits): a single bf16 rounding of either
// would move scores or weights by ~2^-9 relative, enough for errors of a few
// 1e-3 in the output at short lengths.

#include "kvc_internal.h"
#include "kvc_device.h"
#include "kvc_mfma_common.h"

namespace kvc {

namespace {

using namespace mfma;

constexpr int kNW = 4;   // waves per workgroup

// Attended length of sequence b, clamped to [0, max_seq_len]; a step whose
// slot lies outside the cache attends over nothing.
__device__ __forceinline__ int mla_len_lane(const MlaParams& p, int b) {
    int L;
    if (p.positions) {
        const int pos = p.positions[b];
        L = (pos >= 0 && pos < p.T_max) ? pos + 1 : 0;
    } else {
        L = p.seq_lens[b];
    }
    return L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
}
// ... for a b that is the same in every lane (kept in a scalar register)
__device__ __forceinline__ int mla_len(const MlaParams& p, int b) {
    return __builtin_amdgcn_readfirstlane(mla_len_lane(p, b));
}

// hi + lo bf16 pair of 8 floats (hi = RNE(x), lo = RNE(x - hi)).
__device__ __forceinline__ void split8(const float4& a, const float4& b, uint4& hi, uint4& lo) {
    hi.x = pack2_bf16(a.x, a.y);
    hi.y = pack2_bf16(a.z, a.w);
    hi.z = pack2_bf16(b.x, b.y);
    hi.w = pack2_bf16(b.z, b.w);
    lo.x = pack2_bf16(a.x - bf16_lo(hi.x), a.y - bf16_hi(hi.x));
    lo.y = pack2_bf16(a.z - bf16_lo(hi.y), a.w - bf16_hi(hi.y));
    lo.z = pack2_bf16(b.x - bf16_lo(hi.z), b.y - bf16_hi(hi.z));
    lo.w = pack2_bf16(b.z - bf16_lo(hi.w), b.w - bf16_hi(hi.w));
}

// Workgroup barrier that orders nothing by itself: the callers wait for their
// own LDS and direct-load traffic explicitly first.  (The memory clobber keeps
// the compiler from moving memory operations across it.)
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Absorbed queries, q~[b, h, :] = W_uk,h^T q[b, h, :], and (decode step) the
// append of the new rows.  One workgroup per (head, 64 latent columns); wave
// w takes 16 of the columns for every sequence, 16 sequences per product:
//   q~^T[l, b] = sum_i W_uk[h d_k + i, l] q[b, h, i]   A = W_uk,h^T (16 l x 32 i),
//                                                      B = q^T (32 i x 16 b)
// W_uk,h's 64 columns are staged in LDS as rows of i and read transposed.
// ---------------------------------------------------------------------------
template <int DL>
__global__ void __launch_bounds__(256) mla_absorb_kernel(const MlaParams p) {
    const int tid = threadIdx.x;
    if (p.c_new) {
        // the new token's row [c_kv | k_rope] at slot positions[b] (bit copies)
        const uint16_t* cn = static_cast<const uint16_t*>(p.c_new);
        const uint16_t* rn = static_cast<const uint16_t*>(p.r_new);
        uint16_t* cache = static_cast<uint16_t*>(p.cache);
        for (int b = blockIdx.x; b < p.B; b += gridDim.x) {
            const int pos = p.positions[b];
            if (pos < 0 || pos >= p.T_max) continue;
            uint16_t* dst = cache + (static_cast<size_t>(b) * p.T_max + pos) * p.row;
            for (int e = tid; e < p.row; e += blockDim.x)
                dst[e] = e < DL ? cn[static_cast<size_t>(b) * DL + e] : rn[static_cast<size_t>(b) * p.rope_dim + e - DL];
        }
    }
    constexpr int NLB = DL / 64;
    const int h = blockIdx.x / NLB;
    if (h >= p.H) return;
    const int l0 = 64 * (blockIdx.x % NLB);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;

    // W_uk[h d_k + i, l0 .. l0 + 63]: d_k rows of 128 bytes
    __shared__ uint4 wt[512 * 8];
    const uint16_t* wk = static_cast<const uint16_t*>(p.w_uk) + static_cast<size_t>(h) * p.d_k * DL + l0;
    for (int idx = tid; idx < p.d_k * 8; idx += 256) {
        const int i = idx >> 3, c = idx & 7;
        wt[idx] = *reinterpret_cast<const uint4*>(wk + static_cast<size_t>(i) * DL + 8 * c);
    }
    __syncthreads();

    // transposed-read source of this lane: row (i) 4*q4 + s16/4 (+16), columns
    // 16*wave + 4*(s16 % 4) .. +3
    const char* wtb = reinterpret_cast<const char*>(wt);
    const int s16 = lane & 15;
    const int trow = 4 * q4 + s16 / 4;
    const int tcol = 16 * wave + 4 * (s16 % 4);
    const int KK = p.d_k / 32;
    const uint16_t* qb = static_cast<const uint16_t*>(p.q);
    for (int b0 = 0; b0 < p.B; b0 += 16) {
        const int bq = b0 + r16;
        const bool bok = bq < p.B;
        const uint16_t* qrow = qb + (static_cast<size_t>(bok ? bq : 0) * p.H + h) * p.d_k;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kk = 0; kk < KK; ++kk) {
            const int r0 = 32 * kk + trow;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(wtb + r0 * 128 + 2 * tcol));
            const s16x4_t hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(wtb + (r0 + 16) * 128 + 2 * tcol));
            uint4 va;
            va.x = __builtin_bit_cast(uint2, lo).x;
            va.y = __builtin_bit_cast(uint2, lo).y;
            va.z = __builtin_bit_cast(uint2, hi).x;
            va.w = __builtin_bit_cast(uint2, hi).y;
            // B operand: q[b, h, i] for i = 32 kk + 4 q4 + (0..3) and 16 + that
            uint2 qa = *reinterpret_cast<const uint2*>(qrow + 32 * kk + 4 * q4);
            uint2 qc = *reinterpret_cast<const uint2*>(qrow + 32 * kk + 16 + 4 * q4);
            if (!bok) qa = qc = make_uint2(0, 0);
            acc = mfma16(va, make_uint4(qa.x, qa.y, qc.x, qc.y), acc);
        }
        // lane holds q~^T rows l0 + 16 wave + 4 q4 + e of column b
        if (bok)
            *reinterpret_cast<float4*>(p.qt + (static_cast<size_t>(bq) * p.H + h) * DL + l0 + 16 * wave + 4 * q4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

// ---------------------------------------------------------------------------
// The streaming pass (see the top of the file).
// ---------------------------------------------------------------------------
template <int DL, int HB, int NST>
__global__ void __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
mla_decode_kernel(const MlaParams p) {
    constexpr int TT = kMlaTile;          // tokens per tile
    constexpr int DW = DL / kNW;          // latent columns per wave
    constexpr int KKW = DW / 32;          // 32-wide reduction steps of a wave's slice
    constexpr int NBW = DW / 16;          // 16-column blocks of a wave's slice
    constexpr int ROWB = 2 * DL;          // LDS bytes per staged row
    constexpr int STAGE = TT * ROWB;
    constexpr int CPR = DL / 8;           // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;         // rows per wave-wide 16-byte load
    constexpr int LOADS = TT / (kNW * RPI);   // direct loads per thread per tile
    static_assert(CPR >= 16 && LOADS >= 1, "d_latent 128, 256 or 512");
    __shared__ __attribute__((aligned(16))) char st0[STAGE];
    __shared__ __attribute__((aligned(16))) char st1[STAGE];
    __shared__ __attribute__((aligned(16))) char st2[NST > 2 ? STAGE : 16];
    __shared__ f32x4_t sbuf[kNW * HB * 2 * 64];   // partial scores [wave][hb][kb][lane]

    const int wid = blockIdx.x;
    if (wid >= p.n_wg) return;
    const int split = wid % p.n_splits;
    const int unit = wid / p.n_splits;
    const int chunk = unit % p.n_chunks;
    const int b = unit / p.n_chunks;
    const int L = mla_len(p, b);
    const int nsp = L > 0 ? (L + p.split_tokens - 1) / p.split_tokens : 1;
    if (split >= nsp) return;
    const int t_begin = split * p.split_tokens;
    const int t_end = min(L, t_begin + p.split_tokens);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int q4 = lane >> 4;
    const int h0 = chunk * kMlaHeads;     // first head of the chunk
    const int nh = min(kMlaHeads, p.H - h0);

    // Chunk u of tile row r sits at slot u ^ swz(r) of that row in LDS.  The
    // 16 lanes reading one chunk of 16 consecutive rows (score operands) and
    // the 16 lanes of a transposed read (4 rows x 32 bytes) both hit distinct
    // 16-byte bank groups.
    auto swz = [](int r) { return (2 * r + ((r >> 3) & 1)) & 15; };

    // The sequence's rows through a buffer resource ending at row t_end: rows
    // past the split read as zeros without touching memory.
    const uint16_t* cbase = static_cast<const uint16_t*>(p.cache) + static_cast<size_t>(b) * p.T_max * p.row;
    const __amdgpu_buffer_rsrc_t crs = make_uniform_rsrc(cbase, t_end * p.row * 2);
    auto load_tile = [&](int base, char* st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int j = kNW * i + wave;                 // this load's 1 KiB of the stage
            const int rr = RPI * j + lane / CPR;          // row in the tile
            const int u = (lane % CPR) ^ swz(rr);
            lds_void_t* dst = (lds_void_t*)(st + 1024 * j);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, dst, 16, ((base + rr) * p.row + 8 * u) * 2, 0, 0, kNT);
        }
    };

    // Absorbed queries of the chunk's heads, this wave's columns, as hi + lo
    // B operands: lane holds head 16 hb + r16, columns DW*wave + 32 kk + 8 q4 .. +7.
    // Heads past the chunk read zeros.
    const __amdgpu_buffer_rsrc_t qrs =
        make_uniform_rsrc(p.qt + (static_cast<size_t>(b) * p.H + h0) * DL, nh * DL * 4);
    uint4 qh[HB][KKW], ql[HB][KKW];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int kk = 0; kk < KKW; ++kk) {
            const int off = ((16 * hb + r16) * DL + DW * wave + 32 * kk + 8 * q4) * 4;
            const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
            const float4 c = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 16, 0, 0));
            split8(a, c, qh[hb][kk], ql[hb][kk]);
        }

    float m[HB], l[HB];
    f32x4_t o[HB][NBW];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        m[hb] = -kNoMax;
        l[hb] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) o[hb][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int s16 = lane & 15;
    const int tr_row = 4 * q4 + s16 / 4;
    f32x4_t* sw = sbuf + wave * HB * 2 * 64 + lane;

    // One tile: cur holds it; refill receives the tile NST - 1 steps ahead.
    auto body = [&](const char* cur, char* refill, int base) __attribute__((always_inline)) {
        // this thread's loads of the tile have landed (at most NST - 2 later
        // tiles outstanding) and its LDS reads of the previous tile are done;
        // after the barrier that holds for every thread, so the stage the last
        // tile used can be refilled
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NST - 2) * LOADS) & kLgkmZero);
        wg_barrier();
        load_tile(base + (NST - 1) * TT, refill);

        // partial scores over this wave's columns
        uint4 ka[2][KKW];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < KKW; ++kk) {
                const int r = 16 * kb + r16;
                const int u = (DW / 8) * wave + 4 * kk + q4;
                ka[kb][kk] = *reinterpret_cast<const uint4*>(cur + r * ROWB + 16 * (u ^ swz(r)));
            }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < KKW; ++kk) {
                    acc = mfma16(ka[kb][kk], qh[hb][kk], acc);
                    acc = mfma16(ka[kb][kk], ql[hb][kk], acc);
                }
                sw[(hb * 2 + kb) * 64] = acc;
            }
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        wg_barrier();

        // full scores (the four partials added in wave order), scaled to log2
        // units; tokens past the split masked
        float s[HB][8];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const f32x4_t* sp = sbuf + (hb * 2 + kb) * 64 + lane;
                f32x4_t a = sp[0];
#pragma unroll
                for (int w = 1; w < kNW; ++w) a += sp[w * HB * 2 * 64];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = base + 16 * kb + 4 * q4 + e;
                    s[hb][4 * kb + e] = t < t_end ? a[e] * p.scale_log2 : -INFINITY;
                }
            }

        // online softmax, as in the grouped-query kernel: the reference max is
        // moved only when a tile exceeds it by more than 2^kLazy
        uint32_t ph[HB][4], pl[HB][4];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            float mt = s[hb][0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mt = fmaxf(mt, s[hb][e]);
            mt = max_same_head(mt);
            const bool move = mt > m[hb] + kLazy;
            if (__any(move)) {
                const float m_new = move ? mt : m[hb];
                const float alpha = fast_exp2(m[hb] - m_new);
                m[hb] = m_new;
                l[hb] *= alpha;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) o[hb][nb] *= alpha;
            }
            float pr[8], ps = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pr[e] = fast_exp2(s[hb][e] - m[hb]);
                ps += pr[e];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ph[hb][i] = pack2_bf16(pr[2 * i], pr[2 * i + 1]);
                pl[hb][i] = pack2_bf16(pr[2 * i] - bf16_lo(ph[hb][i]), pr[2 * i + 1] - bf16_hi(ph[hb][i]));
            }
            l[hb] += ps;
        }

        // X^T += C^T P^T over this wave's column blocks
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int u = (DW / 8) * wave + 2 * nb + (s16 % 4) / 2;
            const int r0 = tr_row, r1 = tr_row + 16;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)(cur + r0 * ROWB + 16 * (u ^ swz(r0)) + 8 * (s16 & 1)));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)(cur + r1 * ROWB + 16 * (u ^ swz(r1)) + 8 * (s16 & 1)));
            uint4 va;
            va.x = __builtin_bit_cast(uint2, lo).x;
            va.y = __builtin_bit_cast(uint2, lo).y;
            va.z = __builtin_bit_cast(uint2, hi).x;
            va.w = __builtin_bit_cast(uint2, hi).y;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                o[hb][nb] = mfma16(va, make_uint4(ph[hb][0], ph[hb][1], ph[hb][2], ph[hb][3]), o[hb][nb]);
                o[hb][nb] = mfma16(va, make_uint4(pl[hb][0], pl[hb][1], pl[hb][2], pl[hb][3]), o[hb][nb]);
            }
        }
    };

    // Software pipeline over NST stages; every tile load is unconditional
    // (past the split it reads zeros without memory traffic), so the waits
    // above count exactly.
    int base = t_begin;
    load_tile(base, st0);
    if constexpr (NST > 2) load_tile(base + TT, st1);
    if (base < t_end) {
        for (;;) {
            if constexpr (NST == 2) {
                body(st0, st1, base);
                base += TT;
                if (base >= t_end) break;
                body(st1, st0, base);
                base += TT;
                if (base >= t_end) break;
            } else {
                body(st0, st2, base);
                base += TT;
                if (base >= t_end) break;
                body(st1, st0, base);
                base += TT;
                if (base >= t_end) break;
                body(st2, st1, base);
                base += TT;
                if (base >= t_end) break;
            }
        }
    }
    // every direct load has landed before the workgroup ends (its LDS is
    // handed to the next workgroup)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // Epilogue: a whole sequence in one split writes x = X / l; several
    // splits write their (m, l, X) partials.  The wave writes its columns.
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        l[hb] = sum_same_head(l[hb]);
        const int hh = 16 * hb + r16;
        if (hh >= nh) continue;
        const size_t bh = static_cast<size_t>(b) * p.H + h0 + hh;
        if (nsp == 1) {
            const float inv = l[hb] > 0.0f ? 1.0f / l[hb] : 0.0f;
            float* dst = p.ctx + bh * DL + DW * wave + 4 * q4;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                *reinterpret_cast<float4*>(dst + 16 * nb) =
                    make_float4(o[hb][nb][0] * inv, o[hb][nb][1] * inv, o[hb][nb][2] * inv, o[hb][nb][3] * inv);
        } else {
            float* dst = p.ws_part + (bh * p.n_splits + split) * DL + DW * wave + 4 * q4;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
                *reinterpret_cast<float4*>(dst + 16 * nb) =
                    make_float4(o[hb][nb][0], o[hb][nb][1], o[hb][nb][2], o[hb][nb][3]);
            if (wave == 0 && q4 == 0) p.ws_ml[bh * p.n_splits + split] = make_float2(m[hb], l[hb]);
        }
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the splits of one (sequence, head): x = sum_s 2^(m_s -
// M) X_s / sum_s 2^(m_s - M) l_s.  One thread per 4 latent columns.
// ---------------------------------------------------------------------------
template <int DL>
__global__ void __launch_bounds__(DL / 4) mla_merge_kernel(const MlaParams p) {
    const int bh = blockIdx.x;
    const int b = bh / p.H;
    const int L = mla_len(p, b);
    const int nsp = L > 0 ? (L + p.split_tokens - 1) / p.split_tokens : 1;
    if (nsp <= 1) return;                 // written by the streaming pass
    const float2* ml = p.ws_ml + static_cast<size_t>(bh) * p.n_splits;
    float M = -INFINITY;
    for (int s = 0; s < nsp; ++s) M = fmaxf(M, ml[s].x);
    const int c = 4 * threadIdx.x;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float lam = 0.0f;
    const float* part = p.ws_part + static_cast<size_t>(bh) * p.n_splits * DL + c;
    for (int s = 0; s < nsp; ++s) {
        const float2 v = ml[s];
        const float f = fast_exp2(v.x - M);
        const float4 x = *reinterpret_cast<const float4*>(part + static_cast<size_t>(s) * DL);
        acc.x = fmaf(x.x, f, acc.x);
        acc.y = fmaf(x.y, f, acc.y);
        acc.z = fmaf(x.z, f, acc.z);
        acc.w = fmaf(x.w, f, acc.w);
        lam = fmaf(v.y, f, lam);
    }
    const float inv = lam > 0.0f ? 1.0f / lam : 0.0f;
    *reinterpret_cast<float4*>(p.ctx + static_cast<size_t>(bh) * DL + c) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// ---------------------------------------------------------------------------
// Value up-projection, out[b, h, i] = W_uv[h d_k + i, :] . x[b, h, :] +
// b_uv[h d_k + i].  One workgroup per (head, 64 rows of d_k); wave w takes 16
// rows for every sequence, 16 sequences per product:
//   out^T[i, b] = sum_l W_uv[h d_k + i, l] x[b, h, l]   A = W_uv rows (16 i x 32 l),
//                                                       B = x^T (32 l x 16 b), hi + lo
// ---------------------------------------------------------------------------
template <int DL>
__global__ void __launch_bounds__(256) mla_up_kernel(const MlaParams p) {
    constexpr int KK = DL / 32;
    const int nib = (p.d_k + 63) / 64;
    const int h = blockIdx.x / nib;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int i0 = 64 * (blockIdx.x % nib) + 16 * wave;
    if (h >= p.H || i0 >= p.d_k) return;
    const uint16_t* wrow = static_cast<const uint16_t*>(p.w_uv) + (static_cast<size_t>(h) * p.d_k + i0 + r16) * DL + 8 * q4;
    uint4 wa[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) wa[kk] = *reinterpret_cast<const uint4*>(wrow + 32 * kk);
    float bias[4];
    const uint16_t* bv = static_cast<const uint16_t*>(p.b_uv);
#pragma unroll
    for (int e = 0; e < 4; ++e) bias[e] = bv ? bf16_bits_to_f32(bv[static_cast<size_t>(h) * p.d_k + i0 + 4 * q4 + e]) : 0.0f;
    for (int b0 = 0; b0 < p.B; b0 += 16) {
        const int bq = b0 + r16;
        const bool bok = bq < p.B;
        const float* xr = p.ctx + (static_cast<size_t>(bok ? bq : 0) * p.H + h) * DL + 8 * q4;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            float4 a = *reinterpret_cast<const float4*>(xr + 32 * kk);
            float4 c = *reinterpret_cast<const float4*>(xr + 32 * kk + 4);
            if (!bok) a = c = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            uint4 hi, lo;
            split8(a, c, hi, lo);
            acc = mfma16(wa[kk], hi, acc);
            acc = mfma16(wa[kk], lo, acc);
        }
        if (bok) {
            // a sequence that attends over nothing gives zeros
            const bool empty = mla_len_lane(p, bq) == 0;
            float4 r;
            r.x = empty ? 0.0f : acc[0] + bias[0];
            r.y = empty ? 0.0f : acc[1] + bias[1];
            r.z = empty ? 0.0f : acc[2] + bias[2];
            r.w = empty ? 0.0f : acc[3] + bias[3];
            *reinterpret_cast<float4*>(p.out + (static_cast<size_t>(bq) * p.H + h) * p.d_k + i0 + 4 * q4) = r;
        }
    }
}

// bit copy of the new rows (kvc_append_mla), one workgroup per sequence
template <typename T>
__global__ void __launch_bounds__(256) mla_append_kernel(int B, int DL, int rd, T* cache, int T_max,
                                                         const int32_t* positions, const T* cn, const T* rn) {
    const int b = blockIdx.x;
    if (b >= B) return;
    const int pos = positions[b];
    if (pos < 0 || pos >= T_max) return;
    const int row = DL + rd;
    T* dst = cache + (static_cast<size_t>(b) * T_max + pos) * row;
    for (int e = threadIdx.x; e < row; e += blockDim.x)
        dst[e] = e < DL ? cn[static_cast<size_t>(b) * DL + e] : rn[static_cast<size_t>(b) * rd + e - DL];
}

template <int DL>
hipError_t launch_dl(const MlaParams& p, hipStream_t stream, const KernelTiming& tm) {
    hipLaunchKernelGGL(mla_absorb_kernel<DL>, dim3(p.H * (DL / 64)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(p.n_wg), block(kNW * 64);
    constexpr int NST = 2;
    const int rows = min(p.H, kMlaHeads);
    e = rows <= 16 ? launch_timed(mla_decode_kernel<DL, 1, NST>, grid, block, stream, tm, p)
                   : launch_timed(mla_decode_kernel<DL, 2, NST>, grid, block, stream, tm, p);
    if (e != hipSuccess) return e;
    if (p.n_splits > 1) {
        hipLaunchKernelGGL(mla_merge_kernel<DL>, dim3(p.B * p.H), dim3(DL / 4), 0, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(mla_up_kernel<DL>, dim3(p.H * ((p.d_k + 63) / 64)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaParams& p, hipStream_t stream, const KernelTiming& tm) {
    switch (p.d_latent) {
        case 128: return launch_dl<128>(p, stream, tm);
        case 256: return launch_dl<256>(p, stream, tm);
        case 512: return launch_dl<512>(p, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_append_mla(int elem_bytes, int B, int d_latent, int rope_dim, void* cache, int T_max,
                             const int32_t* positions, const void* c_new, const void* r_new, hipStream_t stream) {
    if (elem_bytes == 2)
        hipLaunchKernelGGL(mla_append_kernel<uint16_t>, dim3(B), dim3(256), 0, stream, B, d_latent, rope_dim,
                           static_cast<uint16_t*>(cache), T_max, positions, static_cast<const uint16_t*>(c_new),
                           static_cast<const uint16_t*>(r_new));
    else
        hipLaunchKernelGGL(mla_append_kernel<uint32_t>, dim3(B), dim3(256), 0, stream, B, d_latent, rope_dim,
                           static_cast<uint32_t*>(cache), T_max, positions, static_cast<const uint32_t*>(c_new),
                           static_cast<const uint32_t*>(r_new));
    return hipGetLastError();
}

}  // namespace kvc
