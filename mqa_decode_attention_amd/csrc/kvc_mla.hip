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

// Bit copy of one new row [c_kv | k_rope] (row = DL + rd elements) into dst by
// nt threads: each pass requests four elements per thread before storing any
// (indices clamped to the row, so the loads need no branch).
template <typename T>
__device__ __forceinline__ void copy_new_row(T* dst, const T* cn, const T* rn, int DL, int rd, int tid, int nt) {
    const int row = DL + rd;
    for (int e0 = tid; e0 < row; e0 += 4 * nt) {
        T v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = min(e0 + k * nt, row - 1);
            v[k] = *(e < DL ? cn + e : rn + (e - DL));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e0 + k * nt < row) dst[e0 + k * nt] = v[k];
    }
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
// W_uk,h's 64 columns (rows of i, read transposed) and the 16 sequences'
// query rows are staged in LDS together, so the products wait on one round
// of global loads.
// ---------------------------------------------------------------------------
template <int DL>
__global__ void __launch_bounds__(256) mla_absorb_kernel(const MlaParams p) {
    const int tid = threadIdx.x;
    constexpr int NLB = DL / 64;
    const int h = blockIdx.x / NLB;
    if (h >= p.H) {
        // workgroups past the products (decode step): the new token's row
        // [c_kv | k_rope] of sequence b at slot positions[b] (bit copies)
        const int b = blockIdx.x - p.H * NLB;
        if (!p.c_new || b >= p.B) return;
        const int pos = p.positions[b];
        if (pos < 0 || pos >= p.T_max) return;
        const uint16_t* cn = static_cast<const uint16_t*>(p.c_new) + static_cast<size_t>(b) * DL;
        const uint16_t* rn = static_cast<const uint16_t*>(p.r_new) + static_cast<size_t>(b) * p.rope_dim;
        uint16_t* dst = static_cast<uint16_t*>(p.cache) + (static_cast<size_t>(b) * p.T_max + pos) * p.row;
        copy_new_row(dst, cn, rn, DL, p.rope_dim, tid, static_cast<int>(blockDim.x));
        return;
    }
    const int l0 = 64 * (blockIdx.x % NLB);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;

    // W_uk[h d_k + i, l0 .. l0 + 63]: d_k rows of 128 bytes; query rows of 16
    // sequences, d_k bf16 each, one 16-byte chunk of padding per row (so the
    // 16 rows read at one offset fall in distinct banks)
    __shared__ uint4 wt[512 * 8];
    __shared__ uint4 qs[16 * 65];
    const int dk8 = p.d_k / 8;
    const int qp = dk8 + 1;               // row pitch of qs in 16-byte chunks
    const uint16_t* wk = static_cast<const uint16_t*>(p.w_uk) + static_cast<size_t>(h) * p.d_k * DL + l0;
    const uint16_t* qb = static_cast<const uint16_t*>(p.q);
    const char* wtb = reinterpret_cast<const char*>(wt);
    const char* qsb = reinterpret_cast<const char*>(qs);
    // transposed-read source of this lane: row (i) 4*q4 + s16/4 (+16), columns
    // 16*wave + 4*(s16 % 4) .. +3
    const int s16 = lane & 15;
    const int trow = 4 * q4 + s16 / 4;
    const int tcol = 16 * wave + 4 * (s16 % 4);
    const int KK = p.d_k / 32;            // <= 16; also the W_uk loads per thread
    const int nq = 16 * dk8;              // 16-byte chunks of 16 query rows (<= 4 per thread)
    for (int b0 = 0; b0 < p.B; b0 += 16) {
        if (b0 > 0) __syncthreads();      // the previous block's reads of qs are done
        // Every global load of the block is issued before the first LDS
        // store (loops with a run-time trip count would wait for each load
        // in turn): the W_uk tile (first block only), then the query rows.
        // (W_uk through a buffer resource ending at row d_k: the loads need no
        // guard, and those past it return zeros without a memory access)
        uint4 wv[16], qv[4];
        if (b0 == 0) {
            const __amdgpu_buffer_rsrc_t wrs = make_uniform_rsrc(wk, ((p.d_k - 1) * DL + 64) * 2);
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int idx = tid + 256 * it;
                wv[it] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, ((idx >> 3) * DL + 8 * (idx & 7)) * 2, 0, 0));
            }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx / dk8, c = idx - r * dk8;
            const int bq = b0 + r;
            qv[it] = (idx < nq && bq < p.B)
                         ? *reinterpret_cast<const uint4*>(qb + (static_cast<size_t>(bq) * p.H + h) * p.d_k + 8 * c)
                         : make_uint4(0, 0, 0, 0);
        }
        if (b0 == 0) {
#pragma unroll
            for (int it = 0; it < 16; ++it)
                if (it < KK) wt[tid + 256 * it] = wv[it];
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx / dk8, c = idx - r * dk8;
            if (idx < nq) qs[r * qp + c] = qv[it];
        }
        __syncthreads();
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const char* qrow = qsb + r16 * qp * 16;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            if (kk < KK) {
                const int r0 = 32 * kk + trow;
                const s16x4_t lo =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(wtb + r0 * 128 + 2 * tcol));
                const s16x4_t hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(wtb + (r0 + 16) * 128 + 2 * tcol));
                uint4 va;
                va.x = __builtin_bit_cast(uint2, lo).x;
                va.y = __builtin_bit_cast(uint2, lo).y;
                va.z = __builtin_bit_cast(uint2, hi).x;
                va.w = __builtin_bit_cast(uint2, hi).y;
                // B operand: q[b, h, i] for i = 32 kk + 4 q4 + (0..3) and 16 + that
                const uint2 qa = *reinterpret_cast<const uint2*>(qrow + 2 * (32 * kk + 4 * q4));
                const uint2 qc = *reinterpret_cast<const uint2*>(qrow + 2 * (32 * kk + 16 + 4 * q4));
                acc = mfma16(va, make_uint4(qa.x, qa.y, qc.x, qc.y), acc);
            }
        }
        // lane holds q~^T rows l0 + 16 wave + 4 q4 + e of column b; stored
        // times the softmax scale in log2 units (the streaming pass then
        // computes scores ready for exp2), already split into the hi + lo
        // bf16 pair that pass feeds to the matrix cores (two planes: every
        // hi part, then every lo part)
        const int bq = b0 + r16;
        const float sc = p.scale_log2;
        if (bq < p.B) {
            const float v0 = acc[0] * sc, v1 = acc[1] * sc, v2 = acc[2] * sc, v3 = acc[3] * sc;
            uint2 hi, lo;
            hi.x = pack2_bf16(v0, v1);
            hi.y = pack2_bf16(v2, v3);
            lo.x = pack2_bf16(v0 - bf16_lo(hi.x), v1 - bf16_hi(hi.x));
            lo.y = pack2_bf16(v2 - bf16_lo(hi.y), v3 - bf16_hi(hi.y));
            uint16_t* qth = reinterpret_cast<uint16_t*>(p.qt);
            const size_t at = (static_cast<size_t>(bq) * p.H + h) * DL + l0 + 16 * wave + 4 * q4;
            *reinterpret_cast<uint2*>(qth + at) = hi;
            *reinterpret_cast<uint2*>(qth + static_cast<size_t>(p.B) * p.H * DL + at) = lo;
        }
    }
}

// ---------------------------------------------------------------------------
// The streaming pass.  One workgroup of NWV waves (two per SIMD) per
// (sequence, chunk of up to 32 heads, token split); the split's rows pass
// through LDS in 32-token tiles (direct loads, NST stages).  Wave w takes
// head block hb = w % HB (16 heads) and column slice cs = w / HB of width
// DW = d_latent / (NWV / HB):
//   * scores: the wave multiplies its column slice of the tile by the same
//     slice of its heads' absorbed queries (S^T = C Q~^T, 16 tokens x 16
//     heads per 16x16x32 product) and leaves the partial sums in LDS; after
//     a barrier the waves of a head block add the partials in slice order,
//     so they hold bit-identical scores and run the same online softmax;
//   * PV: the wave accumulates its heads' X^T over its columns, X^T += C^T
//     P^T, C^T read transposed from the staged tile (ds_read_b64_tr_b16).
// ---------------------------------------------------------------------------
template <int DL, int HB, int NST, int NWV>
__global__ void __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
mla_decode_kernel(const MlaParams p) {
    constexpr int TT = kMlaTile;          // tokens per tile
    constexpr int WPH = NWV / HB;         // waves sharing one 16-head block (column slices)
    constexpr int DW = DL / WPH;          // latent columns per wave
    constexpr int KKW = DW / 32;          // 32-wide reduction steps of a wave's slice
    constexpr int NBW = DW / 16;          // 16-column blocks of a wave's slice
    constexpr int ROWB = 2 * DL;          // LDS bytes per staged row
    constexpr int STAGE = TT * ROWB;
    constexpr int CPR = DL / 8;           // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;         // rows per wave-wide 16-byte load
    constexpr int LOADS = TT / (NWV * RPI);   // direct loads per thread per tile
    static_assert(CPR >= 16 && LOADS >= 1 && KKW >= 1, "d_latent 128, 256 or 512");
    static_assert(NST == 2 || NST == 3, "two or three stages");
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    __shared__ __attribute__((aligned(16))) char st0[STAGE];
    __shared__ __attribute__((aligned(16))) char st1[STAGE];
    __shared__ __attribute__((aligned(16))) char st2[NST > 2 ? STAGE : 16];
    __shared__ f32x4_t sbuf[NWV * 2 * 64];   // partial scores [wave][kb][lane]

    const int wid = blockIdx.x;
    if (wid >= p.n_wg) return;
    const int split = wid % p.n_splits;
    const int unit = wid / p.n_splits;
    const int chunk = unit % p.n_chunks;
    const int b = unit / p.n_chunks;
    const int L = mla_len(p, b);
    const int nsp = L > 0 ? (L + p.split_tokens - 1) / p.split_tokens : 1;
    const int tid = threadIdx.x;
    const int h0 = chunk * kMlaHeads;     // first head of the chunk
    const int nh = min(kMlaHeads, p.H - h0);
    if (split >= nsp) {
        // a split past the sequence's end: (m, l) = (-inf, 0), a weight of 0
        // in the merge, which therefore needs no lengths
        if (tid < nh) p.ws_ml[(static_cast<size_t>(b) * p.H + h0 + tid) * p.n_splits + split] = make_float2(-INFINITY, 0.0f);
        return;
    }
    const int t_begin = split * p.split_tokens;
    const int t_end = min(L, t_begin + p.split_tokens);

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hbw = wave % HB;            // this wave's head block
    const int cs = wave / HB;             // ... and column slice
    const int r16 = lane & 15;
    const int q4 = lane >> 4;

    // Chunk u of tile row r sits at slot u ^ swz(r) of that row in LDS: the 16
    // lanes reading one chunk of 16 consecutive rows (score operands) and the
    // 16 lanes of a transposed read (4 rows x 32 bytes) hit distinct 16-byte
    // bank groups.  (A swizzle spreading 8-row groups instead measured twice
    // the bank-conflict cycles.)
    auto swz = [](int r) { return (2 * r + ((r >> 3) & 1)) & 15; };

    // The sequence's rows through a buffer resource ending at row t_end: rows
    // past the split read as zeros without touching memory.
    const uint16_t* cbase = static_cast<const uint16_t*>(p.cache) + static_cast<size_t>(b) * p.T_max * p.row;
    const __amdgpu_buffer_rsrc_t crs = make_uniform_rsrc(cbase, t_end * p.row * 2);
    auto load_tile = [&](int base, char* st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int j = NWV * i + wave;                 // this load's 1 KiB of the stage
            const int rr = RPI * j + lane / CPR;          // row in the tile
            const int u = (lane % CPR) ^ swz(rr);
            lds_void_t* dst = (lds_void_t*)(st + 1024 * j);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, dst, 16, ((base + rr) * p.row + 8 * u) * 2, 0, 0, kNT);
        }
    };

    // Absorbed queries (already scaled to log2 units and split into hi + lo
    // planes) of the wave's head block and columns, as B operands: lane holds
    // head 16 hbw + r16, columns DW*cs + 32 kk + 8 q4 .. +7.  Heads past the
    // chunk read zeros.
    const uint16_t* qth = reinterpret_cast<const uint16_t*>(p.qt) + (static_cast<size_t>(b) * p.H + h0) * DL;
    const __amdgpu_buffer_rsrc_t qhr = make_uniform_rsrc(qth, nh * DL * 2);
    const __amdgpu_buffer_rsrc_t qlr = make_uniform_rsrc(qth + static_cast<size_t>(p.B) * p.H * DL, nh * DL * 2);
    uint4 qh[KKW], ql[KKW];
#pragma unroll
    for (int kk = 0; kk < KKW; ++kk) {
        const int off = ((16 * hbw + r16) * DL + DW * cs + 32 * kk + 8 * q4) * 2;
        qh[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qhr, off, 0, 0));
        ql[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qlr, off, 0, 0));
    }

    // Running max m (log2 units) and sum l of the lane's head; X^T accumulators.
    // The score products start from -m (in the first column slice), so they
    // produce s - m directly; m starts at 0 and is set by the first tile.
    float m = 0.0f, l = 0.0f;
    f32x4_t o[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) o[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int s16 = lane & 15;
    const int tr_row = 4 * q4 + s16 / 4;

    // One tile: cur holds it; refill receives the tile NST - 1 steps ahead.
    auto body = [&](const char* cur, char* refill, int base, bool first) __attribute__((always_inline)) {
        // this thread's loads of the tile have landed (at most NST - 2 later
        // tiles outstanding) and its LDS reads of the previous tile are done;
        // after the barrier that holds for every thread, so the stage the last
        // tile used can be refilled
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NST - 2) * LOADS) & kLgkmZero);
        wg_barrier();
        load_tile(base + (NST - 1) * TT, refill);

        // partial scores (minus m) over this wave's columns
        f32x4_t acc[2];
        const float init = cs == 0 ? -m : 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            acc[kb] = f32x4_t{init, init, init, init};
            const int r = 16 * kb + r16;
#pragma unroll
            for (int kk = 0; kk < KKW; ++kk) {
                const int u = (DW / 8) * cs + 4 * kk + q4;
                const uint4 ka = *reinterpret_cast<const uint4*>(cur + r * ROWB + 16 * (u ^ swz(r)));
                acc[kb] = mfma16(ka, qh[kk], acc[kb]);
                acc[kb] = mfma16(ka, ql[kk], acc[kb]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sbuf[(wave * 2 + kb) * 64 + lane] = acc[kb];
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        wg_barrier();

        // full scores s - m: the slices' partials added in slice order (the
        // wave's own from its registers), bit-identical in all WPH waves
        float s[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4_t a = cs == 0 ? acc[kb] : sbuf[((0 * HB + hbw) * 2 + kb) * 64 + lane];
#pragma unroll
            for (int c = 1; c < WPH; ++c) a += cs == c ? acc[kb] : sbuf[((c * HB + hbw) * 2 + kb) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * kb + e] = a[e];
        }
        if (base + TT > t_end) {          // last tile: rows past the split masked
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (base + 16 * kb + 4 * q4 + e >= t_end) s[4 * kb + e] = -INFINITY;
        }

        // online softmax.  m moves (and X, l are rescaled) only on the first
        // tile or when a tile exceeds it by more than 2^kLazy
        float mt = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, s[e]);
        mt = max_same_head(mt);
        const bool move = first || mt > kLazy;
        if (__any(move)) {
            const float d = move ? mt : 0.0f;
            m += d;
            if (!first) {
                const float alpha = fast_exp2(-d);
                l *= alpha;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) o[nb] *= alpha;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] -= d;
        }
        float pr[8], ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pr[e] = fast_exp2(s[e]);
            ps += pr[e];
        }
        l += ps;
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ph[i] = pack2_bf16(pr[2 * i], pr[2 * i + 1]);
            pl[i] = pack2_bf16(pr[2 * i] - bf16_lo(ph[i]), pr[2 * i + 1] - bf16_hi(ph[i]));
        }
        const uint4 pb_hi = make_uint4(ph[0], ph[1], ph[2], ph[3]);
        const uint4 pb_lo = make_uint4(pl[0], pl[1], pl[2], pl[3]);

        // X^T += C^T P^T over this wave's column blocks
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int u = (DW / 8) * cs + 2 * nb + (s16 % 4) / 2;
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
            o[nb] = mfma16(va, pb_hi, o[nb]);
            o[nb] = mfma16(va, pb_lo, o[nb]);
        }
    };

    // Software pipeline over NST stages; every tile load is unconditional
    // (past the split it reads zeros without memory traffic), so the waits
    // above count exactly.
    int base = t_begin;
    load_tile(base, st0);
    if constexpr (NST > 2) load_tile(base + TT, st1);
    if (base < t_end) {
        bool first = true;
        for (;;) {
            if constexpr (NST == 2) {
                body(st0, st1, base, first);
                first = false;
                if ((base += TT) >= t_end) break;
                body(st1, st0, base, false);
                if ((base += TT) >= t_end) break;
            } else {
                body(st0, st2, base, first);
                first = false;
                if ((base += TT) >= t_end) break;
                body(st1, st0, base, false);
                if ((base += TT) >= t_end) break;
                body(st2, st1, base, false);
                if ((base += TT) >= t_end) break;
            }
        }
    }
    // every direct load has landed before the workgroup ends (its LDS is
    // handed to the next workgroup)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // Epilogue: the split's (m, l, X) partials, each wave its columns of its
    // head block (a split that saw no token leaves m = 0, l = 0, X = 0).
    l = sum_same_head(l);
    const int hh = 16 * hbw + r16;
    if (hh < nh) {
        const size_t bh = static_cast<size_t>(b) * p.H + h0 + hh;
        float* dst = p.ws_part + (bh * p.n_splits + split) * DL + DW * cs + 4 * q4;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            *reinterpret_cast<float4*>(dst + 16 * nb) = make_float4(o[nb][0], o[nb][1], o[nb][2], o[nb][3]);
        if (cs == 0 && q4 == 0) p.ws_ml[bh * p.n_splits + split] = make_float2(m, l);
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the splits: x[b, h, :] = sum_s 2^(m_s - M) X_s /
// sum_s 2^(m_s - M) l_s, one workgroup of d_latent / 4 threads per (sequence,
// head), 4 columns per thread.  Each chunk of 16 splits' (m, l) pairs and
// partials is requested at once; splits past a sequence's end carry m = -inf
// (weight 0) and are skipped by a select (their partials are not written and
// may hold anything).
// ---------------------------------------------------------------------------
template <int DL>
__global__ void __launch_bounds__(DL / 4) mla_merge_kernel(const MlaParams p) {
    const size_t bh = blockIdx.x;
    const int c = 4 * threadIdx.x;
    const float2* ml = p.ws_ml + bh * p.n_splits;
    const float* part = p.ws_part + bh * p.n_splits * DL + c;
    float M = -INFINITY, lam = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = 0; s0 < p.n_splits; s0 += 16) {
        float2 v[16];
        float4 xp[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bool in = s0 + j < p.n_splits;
            v[j] = in ? ml[s0 + j] : make_float2(-INFINITY, 0.0f);
            xp[j] = in ? *reinterpret_cast<const float4*>(part + static_cast<size_t>(s0 + j) * DL)
                       : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < 16; ++j) Mc = fmaxf(Mc, v[j].x);
        const float a = Mc > M ? fast_exp2(M - Mc) : 1.0f;   // rescale of the earlier chunks
        acc.x *= a; acc.y *= a; acc.z *= a; acc.w *= a;
        lam *= a;
        M = Mc;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float f = fast_exp2(v[j].x - M);
            const bool use = f > 0.0f;
            acc.x = use ? fmaf(xp[j].x, f, acc.x) : acc.x;
            acc.y = use ? fmaf(xp[j].y, f, acc.y) : acc.y;
            acc.z = use ? fmaf(xp[j].z, f, acc.z) : acc.z;
            acc.w = use ? fmaf(xp[j].w, f, acc.w) : acc.w;
            lam = use ? fmaf(v[j].y, f, lam) : lam;
        }
    }
    const float inv = lam > 0.0f ? 1.0f / lam : 0.0f;
    *reinterpret_cast<float4*>(p.ctx + bh * DL + c) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// ---------------------------------------------------------------------------
// Value up-projection, out[b, h, i] = W_uv[h d_k + i, :] . x[b, h, :] +
// b_uv[h d_k + i].  One workgroup of four waves per (head, 16 rows of d_k),
// 16 sequences per product:
//   out^T[i, b] = sum_l W_uv[h d_k + i, l] x[b, h, l]   A = W_uv rows (16 i x 32 l),
//                                                       B = x^T (32 l x 16 b), hi + lo
// Wave w takes the latent columns of a quarter of the 32-wide steps, so each
// wave has a quarter of the loads in flight; the four partial products are
// added through LDS in wave order (deterministic).  Each row of W_uv is read
// once per step.
// ---------------------------------------------------------------------------
template <int DL>
__global__ void __launch_bounds__(256) mla_up_kernel(const MlaParams p) {
    constexpr int KK = DL / 32;
    constexpr int KW = KK / 4;            // 32-wide steps per wave
    static_assert(KW >= 1 && KK % 4 == 0, "d_latent a multiple of 128");
    __shared__ f32x4_t part[3][64];       // waves 1..3's partial products
    const int nib = p.d_k / 16;
    const int h = blockIdx.x / nib;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int i0 = 16 * (blockIdx.x - h * nib);
    if (h >= p.H) return;
    const int k0 = wave * KW;             // this wave's first 32-wide step
    const uint16_t* wrow =
        static_cast<const uint16_t*>(p.w_uv) + (static_cast<size_t>(h) * p.d_k + i0 + r16) * DL + 8 * q4 + 32 * k0;
    uint4 wa[KW];
#pragma unroll
    for (int kk = 0; kk < KW; ++kk) wa[kk] = *reinterpret_cast<const uint4*>(wrow + 32 * kk);
    // the bias, read unconditionally (from W_uv when there is none, then
    // replaced by 0) so that no branch separates the loads from each other
    const uint16_t* bv = static_cast<const uint16_t*>(p.b_uv);
    const uint16_t* bsrc = bv ? bv + static_cast<size_t>(h) * p.d_k + i0 + 4 * q4 : wrow;
    uint16_t braw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) braw[e] = bsrc[e];
    for (int b0 = 0; b0 < p.B; b0 += 16) {
        const int bq = b0 + r16;
        const bool bok = bq < p.B;
        const float* xr = p.ctx + (static_cast<size_t>(bok ? bq : 0) * p.H + h) * DL + 8 * q4 + 32 * k0;
        // all of the block's x pieces requested at once, then its length
        float4 xa[KW], xc[KW];
#pragma unroll
        for (int kk = 0; kk < KW; ++kk) {
            xa[kk] = *reinterpret_cast<const float4*>(xr + 32 * kk);
            xc[kk] = *reinterpret_cast<const float4*>(xr + 32 * kk + 4);
        }
        const bool empty = !bok || mla_len_lane(p, bok ? bq : b0) == 0;   // length 0: zeros
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KW; ++kk) {
            float4 a = xa[kk], c = xc[kk];
            if (!bok) a = c = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            uint4 xh, xl;
            split8(a, c, xh, xl);
            acc = mfma16(wa[kk], xh, acc);
            acc = mfma16(wa[kk], xl, acc);
        }
        if (wave > 0) part[wave - 1][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            const f32x4_t r4 = ((acc + part[0][lane]) + part[1][lane]) + part[2][lane];
            float bias[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bias[e] = bv ? bf16_bits_to_f32(braw[e]) : 0.0f;
            if (bok) {
                float4 r;
                r.x = empty ? 0.0f : r4[0] + bias[0];
                r.y = empty ? 0.0f : r4[1] + bias[1];
                r.z = empty ? 0.0f : r4[2] + bias[2];
                r.w = empty ? 0.0f : r4[3] + bias[3];
                *reinterpret_cast<float4*>(p.out + (static_cast<size_t>(bq) * p.H + h) * p.d_k + i0 + 4 * q4) = r;
            }
        }
        __syncthreads();
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
    T* dst = cache + (static_cast<size_t>(b) * T_max + pos) * (DL + rd);
    copy_new_row(dst, cn + static_cast<size_t>(b) * DL, rn + static_cast<size_t>(b) * rd, DL, rd,
                 static_cast<int>(threadIdx.x), static_cast<int>(blockDim.x));
}

// The streaming kernel: eight waves (two per SIMD), or four where an
// eighth of the latent width would be narrower than one 32-wide step; two
// stages (a third measured no faster, as did four waves at d_latent 512).
template <int DL, int HB>
hipError_t launch_main(const MlaParams& p, hipStream_t stream, const KernelTiming& tm) {
    const dim3 grid(p.n_wg);
    if constexpr (DL / (8 / HB) >= 32)
        return launch_timed(mla_decode_kernel<DL, HB, 2, 8>, grid, dim3(8 * 64), stream, tm, p);
    else
        return launch_timed(mla_decode_kernel<DL, HB, 2, 4>, grid, dim3(4 * 64), stream, tm, p);
}

template <int DL>
hipError_t launch_dl(const MlaParams& p, hipStream_t stream, const KernelTiming& tm) {
    hipLaunchKernelGGL(mla_absorb_kernel<DL>, dim3(p.H * (DL / 64) + (p.c_new ? p.B : 0)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rows = min(p.H, kMlaHeads);
    e = rows <= 16 ? launch_main<DL, 1>(p, stream, tm) : launch_main<DL, 2>(p, stream, tm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_merge_kernel<DL>, dim3(p.B * p.H), dim3(DL / 4), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_up_kernel<DL>, dim3(p.H * (p.d_k / 16)), dim3(256), 0, stream, p);
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
