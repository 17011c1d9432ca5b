// kvc_mfma_common.h - device helpers shared by the matrix-core decode kernels
// (bf16 cache: kvc_decode_mfma.hip; uint8 quantized cache: kvc_decode_u8.hip).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "kvc_device.h"

namespace kvc {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cache policy of the K and V tile loads: non-temporal.  The cache is read
// once per step, and on this part streaming reads with the nt bit run at
// about 7.1 TB/s against about 6.2 TB/s with the default policy (same
// access pattern, measured with the library's read probe).
constexpr int kNT = 2;

// The running max is moved only when a tile exceeds it by more than this many
// powers of two (so weights stay <= 2^8 and rescales become rare).
constexpr float kLazy = 8.0f;

// Start of the running max (the largest finite float): below every real score.
constexpr float kNoMax = 3.402823466e38f;

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: A gives lane l the 4 values of row (l % 16) at
// reduction slots 4*(l/16) .. +3, B the 4 values of column (l % 16) at the
// same slots; the results land as in the 16x16x32 product.
__device__ __forceinline__ f32x4_t mfma16k16(const s16x4_t& a, const uint2& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Two float32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and one that waits for every LDS (and scalar memory) operation.
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);

// c ? a : b on values (a conditional between two uint4 lvalues would select
// an address, which forces register arrays into memory).
__device__ __forceinline__ uint4 select4(bool c, const uint4& a, const uint4& b) {
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// Buffer resource from values that are the same in every lane; readfirstlane
// keeps them in scalar registers, so the compiler never needs a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_uniform_rsrc(const void* base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void* ua = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ua, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Lanes l, l^16, l^32, l^48 hold the same query head: reduce over them.
__device__ __forceinline__ float max_same_head(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float sum_same_head(float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

// Cache policy of device-scope buffer accesses (sc1): coherent across the
// XCDs without any cache flush - the split partials one workgroup writes and
// another merges in the same launch.
constexpr int kDevScope = 16;

// Merge of one unit's splits, run by the split that arrived last once every
// split's partial rows went out as device-scope stores: M = max_s m_s,
// w_s = 2^(m_s - M), out = sum_s w_s acc_s / sum_s w_s l_s, the splits in
// order, MB of them requested at a time (their max folded into the running
// one).  rows: output rows of the unit; row_of(r): the output row index of its
// row r; part_of(r, s): the index of split s's partial row for it (the
// partial rows are D floats each in ws_part, their (m, l) pairs in ws_ml).
// One thread per 16-byte column chunk of a row, bf16 output.
template <int D, typename RowOf, typename PartOf>
__device__ __forceinline__ void merge_split_rows(const DecodeParams& p, __amdgpu_buffer_rsrc_t part_rs,
                                                 __amdgpu_buffer_rsrc_t ml_rs, int rows, int nsp, RowOf row_of,
                                                 PartOf part_of) {
    constexpr int NCH = D / 4;
    constexpr int MB = 8;
    for (int idx = threadIdx.x; idx < rows * NCH; idx += blockDim.x) {
        const int c = 4 * (idx % NCH);
        const int gr = idx / NCH;
        const size_t bh = row_of(gr);
        float M = -INFINITY, Ls = 0.0f;
        float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int s0 = 0; s0 < nsp; s0 += MB) {
            float mv[MB], lv[MB];
            float4 pv[MB];
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                if (s0 + u < nsp) {
                    const size_t pr = part_of(gr, s0 + u);
                    const float2 m2 = __builtin_bit_cast(
                        float2, __builtin_amdgcn_raw_buffer_load_b64(ml_rs, static_cast<int>(pr * 8), 0, kDevScope));
                    mv[u] = m2.x;
                    lv[u] = m2.y;
                    pv[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           part_rs, static_cast<int>((pr * D + c) * 4), 0, kDevScope));
                }
            }
            float Mb = M;
#pragma unroll
            for (int u = 0; u < MB; ++u)
                if (s0 + u < nsp) Mb = fmaxf(Mb, mv[u]);
            // (split maxima are finite, so after the first batch M is too)
            const float r = s0 == 0 ? 0.0f : fast_exp2(M - Mb);
            A.x *= r;
            A.y *= r;
            A.z *= r;
            A.w *= r;
            Ls *= r;
            M = Mb;
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                if (s0 + u < nsp) {
                    const float w = fast_exp2(mv[u] - M);
                    A.x = fmaf(w, pv[u].x, A.x);
                    A.y = fmaf(w, pv[u].y, A.y);
                    A.z = fmaf(w, pv[u].z, A.z);
                    A.w = fmaf(w, pv[u].w, A.w);
                    Ls = fmaf(w, lv[u], Ls);
                }
            }
        }
        const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
        uint2 packed;
        packed.x = static_cast<uint32_t>(f32_to_bf16_rne(A.x * inv)) |
                   (static_cast<uint32_t>(f32_to_bf16_rne(A.y * inv)) << 16);
        packed.y = static_cast<uint32_t>(f32_to_bf16_rne(A.z * inv)) |
                   (static_cast<uint32_t>(f32_to_bf16_rne(A.w * inv)) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + bh * D + c) = packed;
    }
}

// ---------------------------------------------------------------------------
// Balanced schedule of the streaming kernels (paged pools with ragged
// lengths).  Sequence b holds n_b = ceil(L_b / STEP) loop steps (at least
// one, so that an empty sequence still writes its zero rows) for each of its
// H_kv units (b, j); the units' steps, in unit order, form one list of T
// steps, and workgroup w of N takes steps [w T / N, (w + 1) T / N): every
// workgroup streams the same number of steps (within one) whatever the
// lengths, and all of them start at once.  N is the planned count, or T when
// there are fewer steps, so that every range holds a step.  A range crosses
// units, so a workgroup runs its split body once per segment (a unit's steps
// inside its range); a unit several workgroups share is merged by the last of
// them to finish, from partial rows each writes to one of two slots of its
// own: slot 0 for its first segment, slot 1 for its last.
// ---------------------------------------------------------------------------

// LDS of the schedule: per-sequence step prefix, lengths, new-token slots.
struct BalLds {
    int pre[kBalMaxB + 1];
    int len[kBalMaxB];
    int pos[kBalMaxB];
    int misc[8];          // per-wave totals; [7]: the sequence holding the first step
};

// Every thread of the workgroup (NT of them, NT * PER >= kBalMaxB) reads PER
// lengths, then the workgroup scans them.  Returns false when this workgroup
// takes no steps (it may return at once).  FUSED: lengths from the new
// tokens' positions (their slots kept for the append).
template <int NT, int STEP, bool FUSED>
__device__ __forceinline__ bool bal_setup(const DecodeParams& p, int wid, BalLds& s) {
    constexpr int PER = kBalMaxB / NT;
    static_assert(PER * NT == kBalMaxB && NT / 64 <= 7, "schedule layout");
    const int tid = threadIdx.x;
    int nst[PER];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int bb = tid * PER + k;
        int n = 0;
        if (bb < p.B) {
            const int ps = FUSED ? p.positions[bb] : 0;
            const int Lb = FUSED ? len_from_position(p, ps) : attended_len(p, bb);
            s.len[bb] = Lb;
            if constexpr (FUSED) s.pos[bb] = ps;
            n = Lb > 0 ? (Lb + STEP - 1) / STEP : 1;
        }
        nst[k] = n;
        sum += n;
    }
    // exclusive prefix over the threads: inside each wave, then over the
    // waves' totals
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if ((tid & 63) >= o) inc += v;
    }
    if ((tid & 63) == 63) s.misc[tid >> 6] = inc;
    __syncthreads();
    int ex = inc - sum, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int v = s.misc[w];
        ex += w < (tid >> 6) ? v : 0;
        tot += v;
    }
    tot = __builtin_amdgcn_readfirstlane(tot);
    const long long T = static_cast<long long>(tot) * p.H_kv;
    const int nwg = T < p.n_wg ? static_cast<int>(T) : p.n_wg;
    const long long s0 = static_cast<long long>(wid) * T / nwg;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int bb = tid * PER + k;
        if (bb < p.B) {
            s.pre[bb] = ex;
            if (static_cast<long long>(ex) * p.H_kv <= s0 && s0 < static_cast<long long>(ex + nst[k]) * p.H_kv)
                s.misc[7] = bb;
        }
        ex += nst[k];
    }
    if (tid == 0) s.pre[p.B] = tot;
    __syncthreads();
    return wid < nwg;
}

// One segment of the schedule.
struct BalSeg {
    int unit;             // b * H_kv + j
    int b, nsp, split;    // the unit's workgroups, this one's index among them
    int L, pos;           // the sequence's attended length, new-token slot (FUSED)
    int t_begin, t_end;   // tokens of the segment
    int wf, slot0;        // the unit's first workgroup, the slot of its partial
    size_t row;           // first partial row of this segment (rows of G)
};

// Segment it of workgroup wid (false past its range).  Everything is derived
// again from LDS and the iteration count, so no state of the schedule stays
// live through the split body between segments.
template <int STEP, bool FUSED>
__device__ __forceinline__ bool bal_segment(const DecodeParams& p, int wid, int it, const BalLds& s, BalSeg& sg) {
    const int tot = __builtin_amdgcn_readfirstlane(s.pre[p.B]);
    const long long T = static_cast<long long>(tot) * p.H_kv;
    const int nwg = T < p.n_wg ? static_cast<int>(T) : p.n_wg;
    const long long s0 = static_cast<long long>(wid) * T / nwg;
    const long long s1 = static_cast<long long>(wid + 1) * T / nwg;
    auto unit_start = [&](int b_, int j_, int& n_) -> long long {   // first step of unit (b_, j_); n_: its steps
        const int pre = __builtin_amdgcn_readfirstlane(s.pre[b_]);
        n_ = __builtin_amdgcn_readfirstlane(s.pre[b_ + 1]) - pre;
        return static_cast<long long>(p.H_kv) * pre + static_cast<long long>(j_) * n_;
    };
    int n0;
    const int b0 = __builtin_amdgcn_readfirstlane(s.misc[7]);
    const long long sb0 = unit_start(b0, 0, n0);
    const int u = b0 * p.H_kv + static_cast<int>((s0 - sb0) / n0) + it;
    if (u >= p.B * p.H_kv) return false;
    const int bq = u / p.H_kv, jj = u - bq * p.H_kv;
    int nb;
    const long long ub = unit_start(bq, jj, nb);                   // the unit's steps [ub, ue)
    if (ub >= s1) return false;
    const long long ue = ub + nb;
    const long long sa = ub > s0 ? ub : s0;                        // this segment: [sa, se)
    const long long se = ue < s1 ? ue : s1;
    // workgroup holding step x: the last w with w T / N <= x
    auto w_of = [&](long long x) { return static_cast<int>(((x + 1) * nwg - 1) / T); };
    sg.wf = w_of(ub);
    sg.unit = u;
    sg.b = bq;
    sg.nsp = w_of(ue - 1) - sg.wf + 1;
    sg.split = wid - sg.wf;
    sg.L = __builtin_amdgcn_readfirstlane(s.len[bq]);
    sg.pos = FUSED ? __builtin_amdgcn_readfirstlane(s.pos[bq]) : 0;
    sg.t_begin = static_cast<int>(sa - ub) * STEP;
    sg.t_end = min(static_cast<int>(se - ub) * STEP, sg.L);
    // the unit's first partial is its first workgroup's second segment when
    // that workgroup's range starts before the unit
    sg.slot0 = static_cast<long long>(sg.wf) * T / nwg < ub ? 1 : 0;
    sg.row = static_cast<size_t>(2 * wid + (it == 0 ? 0 : 1)) * p.G;
    return true;
}

// Partial row of output row gr of split sp of the segment's unit.
__device__ __forceinline__ size_t bal_part_row(const DecodeParams& p, const BalSeg& sg, int gr, int sp) {
    return static_cast<size_t>(2 * (sg.wf + sp) + (sp == 0 ? sg.slot0 : 0)) * p.G + gr;
}

}  // namespace mfma
}  // namespace kvc
