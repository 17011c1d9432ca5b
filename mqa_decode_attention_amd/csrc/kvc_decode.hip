// kvc_decode.hip - attention of one new token per sequence over its KV cache.
//
// What is computed: for query head h of sequence b, with G = H_q / H_kv and
// KV head j = floor(h / G) ("Grouped-query attention: berbagi KV head di antara
// grup query", nalar.dev, section "Jumlah head menentukan batas grup"),
//     out[b, h] = sum_t softmax_t(scale * q[b, h] . K[b, j, t]) V[b, j, t],  t < L_b.
//
// How (the pages name the idea - exact attention streamed through on-chip
// memory with an online softmax, "Arsitektur Inferensi LLM" (tveniu.com),
// section 5 - but no kernel for this chip):
//  * One workgroup per (sequence, KV head, query-head chunk, token split).
//    All query heads of the chunk are scored against each K row as it is
//    read, so the compact KV of a group is read from HBM once, never expanded
//    per query head ("Traffic cache tetap bergantung pada implementasi", same
//    GQA page).
//  * Each wave streams its own token rows straight into registers with 16-byte
//    loads: LPT lanes cover one row (head_dim elements), 64 / LPT rows per load
//    instruction, so every load instruction reads whole contiguous rows.
//  * Scores: bf16 dot2 (two products per instruction, float32 accumulation)
//    summed over the LPT lanes of a row with DPP.  Softmax is online in the
//    log2 domain: running max m, running sum l, rescaled weighted-value sums.
//  * Waves merge through LDS.  A single split writes the output; otherwise each
//    split writes (m, l, acc) to the workspace and a second, small kernel
//    merges the splits of every (sequence, query head) by their log-sum-exp.
//    (Merging inside the split kernel would need an agent-scope release per
//    workgroup, an L2 write-back that measured far slower than a launch.)
//  * Paged caches: token t of sequence b is read from block
//    table[b][t / block_size], offset t % block_size (PagedKVCache listing,
//    youngju.dev; section 4 of the tveniu.com guide).  A 16-token block of one
//    KV head is 4 KiB contiguous, so rows stay whole.

#include "kvc_internal.h"
#include "kvc_device.h"

namespace kvc {

namespace {

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bfloat16 bits
    static constexpr int kPerVec = 8;  // elements per 16-byte load
};
template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;
};

// Rows of LPT lanes, each lane holding EPL = D / LPT consecutive elements.
template <typename T, int D>
struct Layout {
    static constexpr int EPL = Elem<T>::kPerVec;  // one 16-byte load per lane and row
    static constexpr int LPT = D / EPL;
    static constexpr int TPW = 64 / LPT;          // token rows per load instruction
    static_assert(D % EPL == 0 && LPT >= 1 && LPT <= 64, "unsupported head_dim");
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Start of the running max: the largest finite float, negated.
constexpr float kNoMaxF = 3.402823466e38f;

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t i, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(void* out, size_t i, float x) {
    static_cast<uint16_t*>(out)[i] = f32_to_bf16_rne(x);
}
template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t i, float x) {
    static_cast<float*>(out)[i] = x;
}

// One element of the storage type as float32, and back (round to nearest
// even for bf16), as the append kernel reads and writes them.
template <typename T>
struct Store;
template <>
struct Store<float> {
    __device__ static float load(const float* a, size_t i) { return a[i]; }
    __device__ static void store(float* a, size_t i, float x) { a[i] = x; }
};
template <>
struct Store<uint16_t> {
    __device__ static float load(const uint16_t* a, size_t i) { return bf16_bits_to_f32(a[i]); }
    __device__ static void store(uint16_t* a, size_t i, float x) { a[i] = f32_to_bf16_rne(x); }
};

// Partial dot product of one 16-byte K chunk with one query head's chunk.
template <typename T>
struct Dot;
template <>
struct Dot<uint16_t> {
    // q chunk kept as 4 packed bf16 pairs
    using QReg = uint4;
    __device__ static QReg load_q(const void* q, size_t off) {
        return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + off);
    }
    __device__ static float dot(const uint4& k, const QReg& q) {
        float s = dot2_bf16(k.x, q.x, 0.0f);
        s = dot2_bf16(k.y, q.y, s);
        s = dot2_bf16(k.z, q.z, s);
        return dot2_bf16(k.w, q.w, s);
    }
    // the 8 values of a V chunk as float32
    __device__ static void unpack(const uint4& v, float* f) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
};
template <>
struct Dot<float> {
    using QReg = float4;
    __device__ static QReg load_q(const void* q, size_t off) {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(q) + off);
    }
    __device__ static float dot(const uint4& k, const QReg& q) {
        float s = __builtin_bit_cast(float, k.x) * q.x;
        s = fmaf(__builtin_bit_cast(float, k.y), q.y, s);
        s = fmaf(__builtin_bit_cast(float, k.z), q.z, s);
        return fmaf(__builtin_bit_cast(float, k.w), q.w, s);
    }
    __device__ static void unpack(const uint4& v, float* f) {
        f[0] = __builtin_bit_cast(float, v.x); f[1] = __builtin_bit_cast(float, v.y);
        f[2] = __builtin_bit_cast(float, v.z); f[3] = __builtin_bit_cast(float, v.w);
    }
};

template <typename T, int D, int GC, int U, int NW, bool PAGED>
__global__ void __launch_bounds__(NW * 64)
decode_split_kernel(const DecodeParams p) {
    using Lay = Layout<T, D>;
    constexpr int EPL = Lay::EPL, LPT = Lay::LPT, TPW = Lay::TPW;
    constexpr int TILE = U * TPW;  // tokens per wave iteration
    constexpr int NT = NW * 64;

    __shared__ float sm_acc[NW][GC][D];
    __shared__ float sm_m[NW][GC];
    __shared__ float sm_l[NW][GC];
    // decode step (p.valu_step): the chunk's rotated queries and the new
    // token's rotated key and value, in the storage type
    __shared__ __attribute__((aligned(16))) T sm_q[GC * D];
    __shared__ __attribute__((aligned(16))) T sm_kn[D];
    __shared__ __attribute__((aligned(16))) T sm_vn[D];

    const int wid = xcd_logical_id(blockIdx.x, p.n_wg, p.n_wg_pad);
    if (wid < 0) return;
    const int split = wid % p.n_splits;
    const int unit = wid / p.n_splits;          // (b, j, chunk): one query-head chunk of one group
    const int chunk = unit % p.n_chunks;
    const int bj = unit / p.n_chunks;
    const int b = bj / p.H_kv;
    const int j = bj % p.H_kv;

    const TokenRange tr = token_range(p, attended_len(p, b));
    const int nsp = split_count(p, tr);
    if (split >= nsp) return;
    const int t_begin = tr.org + split * p.split_tokens;
    const int t_end = split_end(p, tr, split, nsp);
    const int t_lo = tr.lo;                     // rows before it (window) are masked, never read

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tg = lane / LPT;                  // token row of this lane within a load
    const int el0 = (lane % LPT) * EPL;         // first head_dim element of this lane
    const int h0 = j * p.G + chunk * GC;        // first query head of the chunk

    // Decode step without a separate append: the workgroup rotates its
    // chunk's queries, and the split holding the new token's slot also that
    // token's key, with the append's operation sequence and rounding (into
    // LDS).  That split reads the new row from LDS in place of the cache
    // row, whose store (chunk 0) nothing in this launch reads back; split 0
    // stores the rotated queries.  A slot outside the cache or the rotation
    // table stores nothing and passes the query through unrotated.
    int pos = -1;
    bool holds = false;
    if (p.valu_step) {
        constexpr int HALF = D / 2;
        pos = p.positions[b];
        const bool pos_ok = pos >= 0 && pos < p.capacity && pos < p.rope_rows;
        // the last split stores the new row whenever its slot is valid; it
        // also reads it from LDS when the row is attended (L = pos + 1 is
        // within max_seq_len, so pos lies in this split)
        const bool own = pos_ok && split == nsp - 1;
        holds = own && pos >= t_begin && pos < t_end;
        auto ld = [](const T* a, int i) { return Store<T>::load(a, i); };
        auto pair_at = [&](int i, int& e0, int& e1) {
            if (p.rope_style == KVC_ROPE_HALF) { e0 = i; e1 = i + HALF; }
            else { e0 = 2 * i; e1 = 2 * i + 1; }
        };
        const T* qsrc = static_cast<const T*>(p.q_raw) + (static_cast<size_t>(b) * p.H_q + h0) * D;
        for (int idx = tid; idx < GC * HALF; idx += NT) {
            const int g = idx / HALF, i = idx % HALF;
            int e0, e1;
            pair_at(i, e0, e1);
            const float x0 = ld(qsrc + g * D, e0), x1 = ld(qsrc + g * D, e1);
            float r0 = x0, r1 = x1;
            if (pos_ok)
                rope_pair(x0, x1, p.rope_cos[static_cast<size_t>(pos) * HALF + i],
                          p.rope_sin[static_cast<size_t>(pos) * HALF + i], r0, r1);
            Store<T>::store(sm_q + g * D, e0, r0);
            Store<T>::store(sm_q + g * D, e1, r1);
        }
        if (own) {
            const T* ksrc = static_cast<const T*>(p.k_new) + (static_cast<size_t>(b) * p.H_kv + j) * D;
            const T* vsrc = static_cast<const T*>(p.v_new) + (static_cast<size_t>(b) * p.H_kv + j) * D;
            for (int i = tid; i < HALF; i += NT) {
                int e0, e1;
                pair_at(i, e0, e1);
                float r0, r1;
                rope_pair(ld(ksrc, e0), ld(ksrc, e1), p.rope_cos[static_cast<size_t>(pos) * HALF + i],
                          p.rope_sin[static_cast<size_t>(pos) * HALF + i], r0, r1);
                Store<T>::store(sm_kn, e0, r0);
                Store<T>::store(sm_kn, e1, r1);
            }
            for (int e = tid; e < D; e += NT) sm_vn[e] = vsrc[e];
        }
        __syncthreads();
        if (split == 0 && p.q_rot_out) {
            T* qdst = static_cast<T*>(p.q_rot_out) + (static_cast<size_t>(b) * p.H_q + h0) * D;
            for (int idx = tid; idx < GC * D; idx += NT) qdst[idx] = sm_q[idx];
        }
        if (own && chunk == 0) {
            const size_t slot = ((static_cast<size_t>(b) * p.H_kv + j) * p.T_max + pos) * D;
            for (int e = tid; e < D; e += NT) {
                static_cast<T*>(const_cast<void*>(p.k))[slot + e] = sm_kn[e];
                static_cast<T*>(const_cast<void*>(p.v))[slot + e] = sm_vn[e];
            }
        }
    }

    typename Dot<T>::QReg qr[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g)
        qr[g] = p.valu_step ? Dot<T>::load_q(sm_q, static_cast<size_t>(g) * D + el0)
                            : Dot<T>::load_q(p.q, (static_cast<size_t>(b) * p.H_q + h0 + g) * D + el0);
    // the new row, for the split that holds it
    uint4 k_new_row = make_uint4(0, 0, 0, 0), v_new_row = make_uint4(0, 0, 0, 0);
    if (holds) {
        k_new_row = *reinterpret_cast<const uint4*>(sm_kn + el0);
        v_new_row = *reinterpret_cast<const uint4*>(sm_vn + el0);
    }

    // The running max starts at the lowest finite float, not at -inf: a tile
    // whose rows are all masked (a window's first rows, rounded down to the
    // split origin) then gives alpha = 2^0 and weights 2^-inf = 0, where a
    // start at -inf would give 2^(-inf + inf) = NaN.
    float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        m[g] = -kNoMaxF;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }

    const T* kbase = static_cast<const T*>(p.k);
    const T* vbase = static_cast<const T*>(p.v);
    const size_t seq_off = PAGED ? 0 : (static_cast<size_t>(b) * p.H_kv + j) * p.T_max * D;
    const int32_t* table = PAGED ? p.block_table + static_cast<size_t>(b) * p.max_blocks_per_seq : nullptr;

    for (int base = t_begin + wave * TILE; base < t_end; base += NW * TILE) {
        uint4 kr[U], vr[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + u * TPW + tg;
            valid[u] = t >= t_lo && t < t_end;
            const int tc = t < t_lo ? t_lo : (t < t_end ? t : t_end - 1);   // only attended rows
            size_t off;
            if constexpr (PAGED) {
                int blk = table[tc / p.block_size];
                blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
                off = ((static_cast<size_t>(blk) * p.H_kv + j) * p.block_size + tc % p.block_size) * D;
            } else {
                off = seq_off + static_cast<size_t>(tc) * D;
            }
            kr[u] = *reinterpret_cast<const uint4*>(kbase + off + el0);
            vr[u] = *reinterpret_cast<const uint4*>(vbase + off + el0);
            if (holds && tc == pos) {
                kr[u] = k_new_row;
                vr[u] = v_new_row;
            }
        }

        float s[U][GC];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                const float part = Dot<T>::dot(kr[u], qr[g]);
                const float full = group_sum<LPT>(part) * p.scale_log2;
                s[u][g] = valid[u] ? full : -INFINITY;
            }

#pragma unroll
        for (int g = 0; g < GC; ++g) {
            float mt = s[0][g];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][g]);
            mt = across_groups_max<LPT>(mt);
            const float m_new = fmaxf(m[g], mt);
            const float alpha = fast_exp2(m[g] - m_new);
            m[g] = m_new;
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) s[u][g] = fast_exp2(s[u][g] - m_new);
        }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            Dot<T>::unpack(vr[u], vf);
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                l[g] += s[u][g];
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(s[u][g], vf[e], acc[g][e]);
            }
        }
    }

    // fold the token rows of the wave together (lanes with equal lane % LPT)
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        l[g] = across_groups_sum<LPT>(l[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = across_groups_sum<LPT>(acc[g][e]);
    }
    if (lane < LPT) {
#pragma unroll
        for (int g = 0; g < GC; ++g)
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_acc[wave][g][el0 + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < GC; ++g) {
            sm_m[wave][g] = m[g];
            sm_l[wave][g] = l[g];
        }
    }
    __syncthreads();

    // merge the waves: split result for each (head, element)
    for (int idx = tid; idx < GC * D; idx += NT) {
        const int g = idx / D;
        const int e = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
        float A = 0.0f, Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = sm_m[w][g];
            const float f = (mw == -kNoMaxF) ? 0.0f : fast_exp2(mw - M);   // a wave that saw no row
            A = fmaf(sm_acc[w][g][e], f, A);
            Ls = fmaf(sm_l[w][g], f, Ls);
        }
        const size_t bh = static_cast<size_t>(b) * p.H_q + h0 + g;
        if (nsp == 1) {
            store_out<T>(p.out, bh * D + e, Ls > 0.0f ? A / Ls : 0.0f);
        } else {
            p.ws_part[(bh * p.n_splits + split) * D + e] = A;
            if (e == 0) p.ws_ml[bh * p.n_splits + split] = make_float2(M, Ls);
        }
    }
}

// Merge of the splits of every (sequence, query head) by their log-sum-exp:
// M = max_s m_s, w_s = 2^(m_s - M), out = sum_s w_s acc_s / sum_s w_s l_s.
// One wave per (sequence, query head).  Lane l reads 16 bytes (columns
// 4 * (l % C4) .. +3, C4 = D / 4) of split pass * SPL + l / C4, so one
// wave-wide load covers SPL = 256 / D splits; the (m, l) pairs and the
// partial rows of the first KU passes are requested together, so a merge of
// up to KU * SPL splits waits for memory once.  Lanes holding the same
// columns are summed at the end (fixed order: the result is deterministic).
template <typename T, int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(const DecodeParams p) {
    constexpr int C4 = D / 4;
    constexpr int SPL = 64 / C4;
    constexpr int KU = 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long long bh = static_cast<long long>(blockIdx.x) * 4 + wave;
    // output row bh = (b * qlen + i) * H_q + h
    if (bh >= static_cast<long long>(p.B) * p.qlen * p.H_q) return;
    const int b = static_cast<int>(bh / (static_cast<long long>(p.qlen) * p.H_q));
    const float2* ml = p.ws_ml + bh * p.n_splits;
    const float4* part = reinterpret_cast<const float4*>(p.ws_part + bh * p.n_splits * D);
    const int c4 = lane % C4;
    const int sub = lane / C4;

    // (split indices past the last are clamped and their weight zeroed, so
    // every load is unconditional and all of them are in flight together)
    float4 pv[KU];
    float2 mv[KU];
    bool live[KU];
    auto fetch = [&](int pass0, int n) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int sp = (pass0 + u) * SPL + sub;
            live[u] = sp < n;
            const int spc = live[u] ? sp : n - 1;
            pv[u] = part[static_cast<size_t>(spc) * C4 + c4];
            mv[u] = ml[spc];
        }
    };
    // The first passes are requested before the sequence's length is known
    // (over all n_splits slots of the workspace; those past the sequence's
    // splits are masked once it is), so the two round trips overlap.
    fetch(0, p.n_splits);
    // (under the compacted schedule the streaming kernel picked the split
    // length on the device and recorded each unit's split count)
    const int nsp = p.compact ? p.ws_nsp[static_cast<long long>(b) * p.H_kv + (bh % p.H_q) / (p.H_q / p.H_kv)]
                              : split_count(p, token_range(p, attended_len(p, b)));
    if (nsp <= 1) return;                        // written directly by the split kernel
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        live[u] = u * SPL + sub < nsp;
        if (!live[u]) {                          // (unwritten slots may hold anything)
            pv[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            mv[u] = make_float2(-INFINITY, 0.0f);
        }
    }
    float M = -INFINITY;
    for (int sp = lane; sp < nsp + 63; sp += 64) M = fmaxf(M, ml[sp < nsp ? sp : nsp - 1].x);
    M = across_groups_max<1>(M);

    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float Ls = 0.0f;
    for (int pass0 = 0;;) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const float w = (!live[u] || mv[u].x == -INFINITY) ? 0.0f : fast_exp2(mv[u].x - M);
            acc.x = fmaf(w, pv[u].x, acc.x);
            acc.y = fmaf(w, pv[u].y, acc.y);
            acc.z = fmaf(w, pv[u].z, acc.z);
            acc.w = fmaf(w, pv[u].w, acc.w);
            if (c4 == 0) Ls = fmaf(w, mv[u].y, Ls);
        }
        pass0 += KU;
        if (pass0 * SPL >= nsp) break;
        fetch(pass0, nsp);
    }
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off, 64);
        acc.y += __shfl_xor(acc.y, off, 64);
        acc.z += __shfl_xor(acc.z, off, 64);
        acc.w += __shfl_xor(acc.w, off, 64);
    }
    Ls = across_groups_sum<1>(Ls);
    if (sub == 0) {
        const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
        const size_t o = static_cast<size_t>(bh) * D + 4 * c4;
        store_out<T>(p.out, o + 0, acc.x * inv);
        store_out<T>(p.out, o + 1, acc.y * inv);
        store_out<T>(p.out, o + 2, acc.z * inv);
        store_out<T>(p.out, o + 3, acc.w * inv);
    }
}

constexpr int kU = 4;
constexpr int kNW = 4;

template <typename T, int D, int GC>
hipError_t launch_tdg(bool paged, const DecodeParams& p, hipStream_t stream, const KernelTiming& tm) {
    const dim3 grid(p.n_wg_pad), block(kNW * 64);
    if (paged) return launch_timed(decode_split_kernel<T, D, GC, kU, kNW, true>, grid, block, stream, tm, p);
    return launch_timed(decode_split_kernel<T, D, GC, kU, kNW, false>, grid, block, stream, tm, p);
}

template <typename T, int D>
hipError_t launch_merge_td(const DecodeParams& p, hipStream_t stream) {
    const long long waves = static_cast<long long>(p.B) * p.qlen * p.H_q;   // output rows
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_merge_t(int d, const DecodeParams& p, hipStream_t stream) {
    switch (d) {
        case 16: return launch_merge_td<T, 16>(p, stream);
        case 32: return launch_merge_td<T, 32>(p, stream);
        case 64: return launch_merge_td<T, 64>(p, stream);
        case 128: return launch_merge_td<T, 128>(p, stream);
        case 256: return launch_merge_td<T, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t launch_td(int gc, bool paged, const DecodeParams& p, hipStream_t stream, const KernelTiming& tm) {
    switch (gc) {
        case 1: return launch_tdg<T, D, 1>(paged, p, stream, tm);
        case 2: return launch_tdg<T, D, 2>(paged, p, stream, tm);
        case 4: return launch_tdg<T, D, 4>(paged, p, stream, tm);
        case 8: return launch_tdg<T, D, 8>(paged, p, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_t(int d, int gc, bool paged, const DecodeParams& p, hipStream_t stream, const KernelTiming& tm) {
    switch (d) {
        case 16: return launch_td<T, 16>(gc, paged, p, stream, tm);
        case 32: return launch_td<T, 32>(gc, paged, p, stream, tm);
        case 64: return launch_td<T, 64>(gc, paged, p, stream, tm);
        case 128: return launch_td<T, 128>(gc, paged, p, stream, tm);
        case 256: return launch_td<T, 256>(gc, paged, p, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(kvc_dtype dtype, int d, int heads_per_wg) {
    const bool dt_ok = dtype == KVC_BF16 || dtype == KVC_F32;
    const bool d_ok = d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
    const bool g_ok = heads_per_wg == 1 || heads_per_wg == 2 || heads_per_wg == 4 || heads_per_wg == 8;
    return dt_ok && d_ok && g_ok;
}

int decode_tile_tokens(kvc_dtype dtype, int d) {
    const int epl = dtype == KVC_BF16 ? 8 : 4;
    return kU * (64 / (d / epl)) * kNW;
}

hipError_t launch_decode_split(kvc_dtype dtype, int d, int heads_per_wg, bool paged,
                               const DecodeParams& p, hipStream_t stream, const KernelTiming& tm) {
    if (dtype == KVC_BF16) return launch_t<uint16_t>(d, heads_per_wg, paged, p, stream, tm);
    return launch_t<float>(d, heads_per_wg, paged, p, stream, tm);
}

hipError_t launch_decode_merge(kvc_dtype dtype, int d, const DecodeParams& p, hipStream_t stream) {
    if (dtype == KVC_BF16) return launch_merge_t<uint16_t>(d, p, stream);
    return launch_merge_t<float>(d, p, stream);
}

}  // namespace kvc
