// kvc_append.hip - store the new token's rotated key and its value as one
// slice along the token axis of the cache, and rotate its query in place.
//
// The cache layout and the "rotate once, store rotated" rule follow the "KV
// Cache" explainer (lensaml.com), step 3; the paged slot (block table entry
// pos / block_size, offset pos % block_size) follows the PagedKVCache listing of
// "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략"
// (youngju.dev) and section 4 of "Arsitektur Inferensi LLM: PagedAttention,
// KV-Cache & Speculative Decoding" (tveniu.com).
//
// The rotation of a pair (x0, x1) by (c, s) is the float32 sequence
//   r0 = (x0*c) - (x1*s),  r1 = (x0*s) + (x1*c)
// with every operation rounded on its own (rope_pair: no fused multiply-add;
// this file is also compiled with -ffp-contract=off), so the stored bits are
// fixed by the inputs alone.

#include "kvc_internal.h"
#include "kvc_device.h"

#pragma clang fp contract(off)

namespace kvc {

namespace {

template <typename T>
struct Store;

template <>
struct Store<float> {
    __device__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ static void store(float* p, size_t i, float x) { p[i] = x; }
};

template <>
struct Store<uint16_t> {
    __device__ static float load(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
    __device__ static void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16_rne(x); }
};

// One thread per (sequence, new token, vector, pair).  Vectors of token bt =
// b * qlen + t, in order: the H_kv keys (rotated into the cache), the H_kv
// values (copied into the cache), then, when q_inout is given, the H_q
// queries (rotated in place, or from q_in into q_inout).  Token t of
// sequence b takes position positions[b] + t.
template <typename T>
__global__ void __launch_bounds__(256) append_kernel(const AppendParams p) {
    const int half = p.d >> 1;
    const int qlen = p.qlen > 0 ? p.qlen : 1;
    const int nvec = 2 * p.H_kv + (p.q_inout ? p.H_q : 0);
    const long long total = static_cast<long long>(p.B) * qlen * nvec * half;
    const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int i = static_cast<int>(idx % half);
    const int vec = static_cast<int>((idx / half) % nvec);
    const int bt = static_cast<int>(idx / (static_cast<long long>(half) * nvec));
    const int b = bt / qlen;

    int e0, e1;
    if (p.rope_style == KVC_ROPE_HALF) { e0 = i; e1 = i + half; }
    else { e0 = 2 * i; e1 = 2 * i + 1; }

    // A token whose slot is invalid stores nothing; a query read from q_in
    // still reaches q_inout, unrotated (as a copy rotated in place is left).
    auto pass_query = [&]() {
        if (p.q_in && vec >= 2 * p.H_kv) {
            const size_t off = (static_cast<size_t>(bt) * p.H_q + (vec - 2 * p.H_kv)) * p.d;
            const T* src = static_cast<const T*>(p.q_in) + off;
            T* dst = static_cast<T*>(p.q_inout) + off;
            dst[e0] = src[e0];
            dst[e1] = src[e1];
        }
    };
    const long long pos_ll = static_cast<long long>(p.positions[b]) + (bt - b * qlen);
    if (pos_ll < 0 || pos_ll >= p.capacity || pos_ll >= p.rope_rows) {
        pass_query();
        return;
    }
    const int pos = static_cast<int>(pos_ll);

    // slot of (b, head j) in the cache, in elements, for head 0; + j * head stride
    size_t slot0;
    size_t head_stride;
    if (p.block_table) {
        const int blk = p.block_table[static_cast<size_t>(b) * p.max_blocks_per_seq + pos / p.block_size];
        if (blk < 0 || blk >= p.num_blocks) {
            pass_query();
            return;
        }
        slot0 = (static_cast<size_t>(blk) * p.H_kv * p.block_size + pos % p.block_size) * p.d;
        head_stride = static_cast<size_t>(p.block_size) * p.d;
    } else {
        // (a ring of T_max slots keeps position pos in slot pos % T_max)
        slot0 = (static_cast<size_t>(b) * p.H_kv * p.T_max + (p.ring ? pos % p.T_max : pos)) * p.d;
        head_stride = static_cast<size_t>(p.T_max) * p.d;
    }

    if (vec >= p.H_kv && vec < 2 * p.H_kv) {  // value: bit copy of both elements
        const int j = vec - p.H_kv;
        const T* src = static_cast<const T*>(p.v_new) + (static_cast<size_t>(bt) * p.H_kv + j) * p.d;
        T* dst = static_cast<T*>(p.v_cache) + slot0 + j * head_stride;
        dst[2 * i] = src[2 * i];
        dst[2 * i + 1] = src[2 * i + 1];
        return;
    }

    const float c = p.rope_cos[static_cast<size_t>(pos) * half + i];
    const float s = p.rope_sin[static_cast<size_t>(pos) * half + i];
    const T* src;
    T* dst;
    if (vec < p.H_kv) {
        src = static_cast<const T*>(p.k_new) + (static_cast<size_t>(bt) * p.H_kv + vec) * p.d;
        dst = static_cast<T*>(p.k_cache) + slot0 + vec * head_stride;
    } else {
        const int h = vec - 2 * p.H_kv;
        const size_t off = (static_cast<size_t>(bt) * p.H_q + h) * p.d;
        dst = static_cast<T*>(p.q_inout) + off;
        src = p.q_in ? static_cast<const T*>(p.q_in) + off : dst;
    }
    const float x0 = Store<T>::load(src, e0);
    const float x1 = Store<T>::load(src, e1);
    float r0, r1;
    rope_pair(x0, x1, c, s, r0, r1);
    Store<T>::store(dst, e0, r0);
    Store<T>::store(dst, e1, r1);
}

// Quantized cache: the new key (rotated as above, kept in float32) and value
// of each (sequence, KV head) become uint8 codes with one (step, zero point)
// pair, following the QuantizedKVCache listing of "KV Cache 최적화 심층 분석:
// GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략" (youngju.dev) with a pair per
// vector: over the vector, step = (max - min) / 255 (taken as 1 when it is 0),
// zero point = -min / step rounded to nearest-even and clamped to [0, 255],
// code = x / step + zero point rounded and clamped to [0, 255]; float32, one
// rounding per operation.  One wave per vector: the H_kv keys, the H_kv
// values, then (q_inout given) the H_q queries, rotated in place as above.
//
// FP8 cache (FMT kQ8E4M3 / kQ8E5M2: the one-byte FP8 caches of "Arsitektur
// Inferensi LLM", tveniu.com, sections 2 and 8, and of the vLLM commands of
// "KV Cache 최적화 심층 분석", youngju.dev): E4M3 codes of x / scale with the
// float32 scale = (largest magnitude over the vector) / 448 (taken as 1 when
// it is 0), so that the largest element lands on +-448; E5M2 codes of x
// itself (scale 1).  Round to nearest even, saturating (fp8_encode); the pair
// stored is (scale, 0).
template <typename T, int FMT>
__global__ void __launch_bounds__(256) append_u8_kernel(const AppendParams p) {
    const int lane = threadIdx.x & 63;
    const int nvec = 2 * p.H_kv + (p.q_inout ? p.H_q : 0);
    const long long gw = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (gw >= static_cast<long long>(p.B) * nvec) return;
    const int vec = static_cast<int>(gw % nvec);
    const int b = static_cast<int>(gw / nvec);
    const int pos = p.positions[b];
    if (pos < 0 || pos >= p.capacity || pos >= p.rope_rows) return;
    const int half = p.d >> 1;

    // row index (in vectors of d elements) of (b, head 0) at slot pos, and the
    // stride between heads
    size_t row0, head_rows;
    if (p.block_table) {
        const int blk = p.block_table[static_cast<size_t>(b) * p.max_blocks_per_seq + pos / p.block_size];
        if (blk < 0 || blk >= p.num_blocks) return;
        row0 = static_cast<size_t>(blk) * p.H_kv * p.block_size + pos % p.block_size;
        head_rows = p.block_size;
    } else {
        row0 = static_cast<size_t>(b) * p.H_kv * p.T_max + (p.ring ? pos % p.T_max : pos);
        head_rows = p.T_max;
    }

    // lane handles pairs i = lane and lane + 64 (d <= 256)
    float x[4];
    int el[4];
    bool has[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = lane + 64 * k;
        has[k] = i < half;
        el[2 * k] = p.rope_style == KVC_ROPE_HALF ? i : 2 * i;
        el[2 * k + 1] = p.rope_style == KVC_ROPE_HALF ? i + half : 2 * i + 1;
    }
    const bool is_key = vec < p.H_kv;
    const bool is_query = vec >= 2 * p.H_kv;
    const int j = is_key ? vec : vec - p.H_kv;
    const T* src;
    if (is_query)
        src = static_cast<const T*>(p.q_in ? p.q_in : p.q_inout) + (static_cast<size_t>(b) * p.H_q + vec - 2 * p.H_kv) * p.d;
    else src = static_cast<const T*>(is_key ? p.k_new : p.v_new) + (static_cast<size_t>(b) * p.H_kv + j) * p.d;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        x[2 * k] = 0.0f;
        x[2 * k + 1] = 0.0f;
        if (!has[k]) continue;
        const float x0 = Store<T>::load(src, el[2 * k]);
        const float x1 = Store<T>::load(src, el[2 * k + 1]);
        if (is_query || is_key) {
            const int i = lane + 64 * k;
            const float c = p.rope_cos[static_cast<size_t>(pos) * half + i];
            const float s = p.rope_sin[static_cast<size_t>(pos) * half + i];
            rope_pair(x0, x1, c, s, x[2 * k], x[2 * k + 1]);
        } else {
            x[2 * k] = x0;
            x[2 * k + 1] = x1;
        }
    }
    if (is_query) {
        T* dst = static_cast<T*>(p.q_inout) + (static_cast<size_t>(b) * p.H_q + vec - 2 * p.H_kv) * p.d;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!has[k]) continue;
            Store<T>::store(dst, el[2 * k], x[2 * k]);
            Store<T>::store(dst, el[2 * k + 1], x[2 * k + 1]);
        }
        return;
    }

    const size_t row = row0 + static_cast<size_t>(j) * head_rows;
    uint8_t* codes = static_cast<uint8_t*>(is_key ? p.k_cache : p.v_cache) + row * p.d;
    float first, second;                  // the vector's pair
    if constexpr (FMT == kQ8Affine) {
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!has[k]) continue;
            mn = fminf(mn, fminf(x[2 * k], x[2 * k + 1]));
            mx = fmaxf(mx, fmaxf(x[2 * k], x[2 * k + 1]));
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, off, 64));
            mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        }
        float step = (mx - mn) / 255.0f;
        step = step == 0.0f ? 1.0f : step;
        const float zp = fminf(fmaxf(rintf(-mn / step), 0.0f), 255.0f);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!has[k >> 1]) continue;
            codes[el[k]] = static_cast<uint8_t>(fminf(fmaxf(rintf(x[k] / step + zp), 0.0f), 255.0f));
        }
        first = step;
        second = zp;
    } else {
        float scale = 1.0f;
        if constexpr (FMT == kQ8E4M3) {
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (!has[k]) continue;
                amax = fmaxf(amax, fmaxf(fabsf(x[2 * k]), fabsf(x[2 * k + 1])));
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
            scale = amax / 448.0f;
            scale = scale == 0.0f ? 1.0f : scale;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!has[k >> 1]) continue;
            codes[el[k]] = static_cast<uint8_t>(fp8_encode<FMT>(x[k] / scale));
        }
        first = scale;
        second = 0.0f;
    }
    if (lane == 0) {
        float* sz = (is_key ? p.k_sz : p.v_sz) + row * 2;
        sz[0] = first;
        sz[1] = second;
    }
}

}  // namespace

hipError_t launch_append_u8(const AppendParams& p, hipStream_t stream) {
    const int nvec = 2 * p.H_kv + (p.q_inout ? p.H_q : 0);
    const long long blocks = (static_cast<long long>(p.B) * nvec + 3) / 4;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    const bool b16 = p.dtype == KVC_BF16;
    switch (p.qfmt) {
        case kQ8Affine:
            if (b16) hipLaunchKernelGGL((append_u8_kernel<uint16_t, kQ8Affine>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((append_u8_kernel<float, kQ8Affine>), grid, block, 0, stream, p);
            break;
        case kQ8E4M3:
            if (b16) hipLaunchKernelGGL((append_u8_kernel<uint16_t, kQ8E4M3>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((append_u8_kernel<float, kQ8E4M3>), grid, block, 0, stream, p);
            break;
        case kQ8E5M2:
            if (b16) hipLaunchKernelGGL((append_u8_kernel<uint16_t, kQ8E5M2>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((append_u8_kernel<float, kQ8E5M2>), grid, block, 0, stream, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
    const int nvec = 2 * p.H_kv + (p.q_inout ? p.H_q : 0);
    const long long total = static_cast<long long>(p.B) * (p.qlen > 0 ? p.qlen : 1) * nvec * (p.d / 2);
    const int threads = 256;
    const long long blocks = (total + threads - 1) / threads;
    if (blocks <= 0) return hipSuccess;
    if (p.dtype == KVC_BF16)
        hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream, p);
    else
        hipLaunchKernelGGL(append_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kvc
