// kvc_device.h - small device helpers shared by the libkvc kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_internal.h"

namespace kvc {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bfloat16 <-> float32.  bf16 is the upper half of an IEEE float32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round float32 to the nearest bfloat16, ties to even (integer form, so the
// result never depends on a hardware rounding mode).  NaN stays a quiet NaN.
// (Written as a select, so no divergent branch is generated.)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x0040u;
    return static_cast<uint16_t>(((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16_rne(lo)) | (static_cast<uint32_t>(f32_to_bf16_rne(hi)) << 16);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 operands and float32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// RoPE rotation of one pair (x0, x1) by (c, s), every operation rounded to
// float32 on its own (no fused multiply-add), so the result is fixed by the
// inputs:  r0 = (x0*c) - (x1*s),  r1 = (x0*s) + (x1*c).
// ---------------------------------------------------------------------------

__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float s, float& r0, float& r1) {
#pragma clang fp contract(off)
    const float a = x0 * c;
    const float b = x1 * s;
    const float e = x0 * s;
    const float f = x1 * c;
    r0 = a - b;
    r1 = e + f;
}

// ---------------------------------------------------------------------------
// Cross-lane exchange inside a 64-wide wavefront.
// DPP controls (GFX9 encoding): quad_perm(a,b,c,d) = a | b<<2 | c<<4 | d<<6,
// row_mirror = 0x140 (lane i <-> 15-i in a row of 16),
// row_half_mirror = 0x141 (lane i <-> 7-i in a half row of 8).
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Value held by lane (lane ^ MASK).  MASK 1, 2 use quad permutes; 4 and 8 use
// mirrors, which pair lanes whose partners cover the same set after the lower
// masks have been folded in (valid inside butterfly reductions only); 16 and
// 32 go through ds_swizzle / bpermute.
template <int MASK>
__device__ __forceinline__ float xor_partner(float x) {
    if constexpr (MASK == 1) return dpp<(1 | (0 << 2) | (3 << 4) | (2 << 6))>(x);
    else if constexpr (MASK == 2) return dpp<(2 | (3 << 2) | (0 << 4) | (1 << 6))>(x);
    else if constexpr (MASK == 4) return dpp<0x141>(x);
    else if constexpr (MASK == 8) return dpp<0x140>(x);
    else return __shfl_xor(x, MASK, 64);
}

// Butterfly sum over groups of W consecutive lanes (W a power of two <= 64):
// every lane of the group ends with the group total.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 2) x += xor_partner<1>(x);
    if constexpr (W >= 4) x += xor_partner<2>(x);
    if constexpr (W >= 8) x += xor_partner<4>(x);
    if constexpr (W >= 16) x += xor_partner<8>(x);
    if constexpr (W >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (W >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// Sum / max over lanes that share (lane % W0) across the wave (strides W0..32):
// folds the 64/W0 lane groups of width W0 together.
template <int W0>
__device__ __forceinline__ float across_groups_sum(float x) {
    if constexpr (W0 <= 1) x += xor_partner<1>(x);
    if constexpr (W0 <= 2) x += xor_partner<2>(x);
    if constexpr (W0 <= 4) x += __shfl_xor(x, 4, 64);
    if constexpr (W0 <= 8) x += __shfl_xor(x, 8, 64);
    if constexpr (W0 <= 16) x += __shfl_xor(x, 16, 64);
    if constexpr (W0 <= 32) x += __shfl_xor(x, 32, 64);
    return x;
}

template <int W0>
__device__ __forceinline__ float across_groups_max(float x) {
    if constexpr (W0 <= 1) x = fmaxf(x, __shfl_xor(x, 1, 64));
    if constexpr (W0 <= 2) x = fmaxf(x, __shfl_xor(x, 2, 64));
    if constexpr (W0 <= 4) x = fmaxf(x, __shfl_xor(x, 4, 64));
    if constexpr (W0 <= 8) x = fmaxf(x, __shfl_xor(x, 8, 64));
    if constexpr (W0 <= 16) x = fmaxf(x, __shfl_xor(x, 16, 64));
    if constexpr (W0 <= 32) x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// One float32 value as an 8-bit floating-point code, from the formats'
// definitions (E4M3: exponent bias 7, 3 mantissa bits, largest finite 448;
// E5M2: bias 15, 2 mantissa bits, largest finite 57344): round to nearest,
// ties to even; results past the largest finite value saturate to it; the
// sign of zero is kept.  (Finite inputs.)
template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode(float x) {
    constexpr int MB = FMT == kQ8E4M3 ? 3 : 2;
    constexpr int BIAS = FMT == kQ8E4M3 ? 7 : 15;
    constexpr uint32_t MAXC = FMT == kQ8E4M3 ? 0x7Eu : 0x7Bu;          // codes of 448 and 57344
    constexpr float VMAX = FMT == kQ8E4M3 ? 448.0f : 57344.0f;
    constexpr float MIN_NORMAL = FMT == kQ8E4M3 ? 0.015625f : 6.103515625e-05f;   // 2^-6, 2^-14
    constexpr float SUB_SCALE = static_cast<float>(1 << (BIAS + MB - 1));         // 1 / subnormal step
    const uint32_t bits = __float_as_uint(x);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = fabsf(x);
    uint32_t mag;
    if (a >= VMAX) {
        mag = MAXC;
    } else if (a < MIN_NORMAL) {
        // multiples of the subnormal step (the scaling is exact); a count of
        // 2^MB is the smallest normal's code
        mag = static_cast<uint32_t>(rintf(a * SUB_SCALE));
    } else {
        const int e = static_cast<int>((bits >> 23) & 0xFFu) - 127;
        uint32_t keep = (bits & 0x7FFFFFu) >> (23 - MB);
        const uint32_t rest = bits & ((1u << (23 - MB)) - 1u);
        const uint32_t halfway = 1u << (22 - MB);
        if (rest > halfway || (rest == halfway && (keep & 1u))) ++keep;
        // (a carry out of the mantissa moves the code to the next binade)
        mag = (static_cast<uint32_t>(e + BIAS) << MB) + keep;
        mag = mag > MAXC ? MAXC : mag;
    }
    return sign | mag;
}

// Workgroup id remap so that consecutive logical ids share one XCD.  The
// hardware hands workgroup i to XCD i % 8; logical id = xcd * (n/8) + i / 8.
// n_pad must be a multiple of 8; ids >= n (padding) return -1.
__device__ __forceinline__ int xcd_logical_id(int hw_id, int n, int n_pad) {
    const int per = n_pad >> 3;
    const int id = (hw_id & 7) * per + (hw_id >> 3);
    return id < n ? id : -1;
}

}  // namespace kvc
