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

}  // namespace mfma
}  // namespace kvc
