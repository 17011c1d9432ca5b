// kvc_decode_mfma.hip - bf16 decode attention on the gfx950 matrix cores.
//
// Same contract as the split kernel in kvc_decode.hip (one workgroup per
// (sequence, KV head, token split); split results merged by their log-sum-exp;
// scores = scale * q . k and out = softmax-weighted V rows, per query head of
// the group g(h) = floor(h / G) - "Grouped-query attention: berbagi KV head di
// antara grup query", nalar.dev, section "Jumlah head menentukan batas grup"),
// but both products of a 32-token tile run as v_mfma_f32_16x16x32_bf16:
//
//   S^T[t, g] = sum_d K[t, d] Q[g, d]        A = K rows (16 tokens x 32 d),
//                                            B = Q^T (32 d x 16 heads)
//   O^T[c, g] += sum_t V[t, c] P[g, t]       A = V^T (16 columns x 32 tokens),
//                                            B = P^T (32 tokens x 16 heads)
//
// Operand layouts (16x16x32, wave64): an A operand gives lane l the 8 values of
// row (l % 16) at reduction slots 8*(l/16) .. +7; a B operand gives lane l the 8
// values of column (l % 16) at the same slots; the 4 results of lane l are rows
// 4*(l/16) .. +3 of column (l % 16).  The reduction slots only have to agree
// between A and B, so any fixed assignment of d (or of tokens) to slots works.
//
// * K rows go from HBM straight into the A operand with 16-byte loads.
// * S^T leaves lane l with one query head (l % 16) and 8 tokens of the tile.
//   That is exactly the B operand P^T of the second product once the tokens
//   are mapped to slots as tok(q, e) = 4q + e (e < 4), 16 + 4q + (e - 4) (e >= 4),
//   q = l / 16, so the probabilities never leave their lane.  The softmax
//   rescale of O^T is lane-local too: O^T also keeps head (l % 16) in lane l.
// * V rows are read with whole-row 16-byte loads, stored row-major in this
//   wave's LDS slice, and read back transposed with ds_read_b64_tr_b16: inside
//   each 16-lane group, output lane 4a+b receives element b of the 8-byte
//   chunks addressed by lanes a, a+4, a+8, a+12.  Pointing source lane s at
//   row tok(q, s/4 [+4]) and columns 16*nb + 4*(s % 4) .. +3 gives each lane 4
//   tokens of one V column - the A operand V^T - with one instruction.
// * Query heads beyond G are zero rows of the B operand; more than 16 heads use
//   several 16-head blocks over the same K/V registers.
// * The probabilities enter the second product as a pair of bf16 operands
//   (hi = bf16(p), lo = bf16(p - hi)), two MFMAs, so p carries about 16
//   significant bits: rounding p once to bf16 alone would leave errors of a
//   few 1e-4 in the output, enough to move it across a bf16 rounding boundary.

#include "kvc_internal.h"
#include "kvc_device.h"

namespace kvc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The running max is moved only when a tile exceeds it by more than this many
// powers of two (so weights stay <= 2^8 and rescales become rare).
constexpr float kLazy = 8.0f;

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two float32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
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

// MODE 0: contiguous cache.  MODE 1: paged, any block size (each row's block
// looked up per lane).  MODE 2: paged with block_size % 16 == 0 and splits
// starting on 32-token boundaries, so every 16-row group of a tile lies in one
// block: one wave-uniform table lookup per group.
template <int D, int HB, int NW, int MODE, bool FUSED>
__global__ void __launch_bounds__(NW * 64)
decode_mfma_kernel(const DecodeParams p, const int32_t* __restrict__ block_table) {
    // (the block table as its own restrict argument: nothing this kernel stores
    // can alias it, so its wave-uniform reads may use scalar loads)
    constexpr bool PAGED = MODE != 0;
    constexpr int KK = D / 32;            // 32-wide d slices per 16-token block
    constexpr int NB = D / 16;            // 16-column blocks of V
    constexpr int TT = 32;                // tokens per wave tile
    constexpr int ROWB = 2 * D;           // LDS bytes per staged V row
    constexpr int STAGE = TT * ROWB;      // LDS bytes of one V tile
    // V tiles are double-buffered per wave; two separate arrays, so the
    // compiler can tell the tile being read from the one being filled.
    __shared__ __attribute__((aligned(16))) char vbuf0[NW * STAGE];
    __shared__ __attribute__((aligned(16))) char vbuf1[NW * STAGE];
    static_assert(NW * STAGE >= NW * 16 * D * 4 && NW * STAGE >= 2 * NW * 16 * 4, "merge area");

    const int wid = xcd_logical_id(blockIdx.x, p.n_wg, p.n_wg_pad);
    if (wid < 0) return;
    const int split = wid % p.n_splits;
    const int unit = wid / p.n_splits;    // b * H_kv + j
    const int b = unit / p.H_kv;
    const int j = unit % p.H_kv;
    const int G = p.G;

    const int L = attended_len(p, b);
    int nsp = (L + p.split_tokens - 1) / p.split_tokens;
    nsp = nsp < 1 ? 1 : nsp;
    if (split >= nsp) return;
    const int t_begin = split * p.split_tokens;
    const int t_end = min(L, t_begin + p.split_tokens);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;            // row/column index inside the operand
    const int q4 = lane >> 4;             // 16-lane group: reduction slots 8*q4 .. +7

    float m[HB], l[HB];
    f32x4_t o[HB][NB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        m[hb] = -INFINITY;
        l[hb] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[hb][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(p.k);
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v);
    const size_t seq_off = PAGED ? 0 : (static_cast<size_t>(b) * p.H_kv + j) * p.T_max * D;
    const int32_t* table = PAGED ? block_table + static_cast<size_t>(b) * p.max_blocks_per_seq : nullptr;
    auto row_off = [&](int t) -> size_t {   // element offset of token t's row (t < L)
        if constexpr (PAGED) {
            int blk = table[t / p.block_size];
            blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
            return ((static_cast<size_t>(blk) * p.H_kv + j) * p.block_size + t % p.block_size) * D;
        } else {
            return seq_off + static_cast<size_t>(t) * D;
        }
    };

    constexpr int LPR = D / 8;            // 16-byte chunks (lanes) per V row
    constexpr int VROWS = 64 / LPR;       // V rows per wave-wide 16-byte load
    constexpr int VLOADS = TT / VROWS;
    // Chunk u of tile row r sits at slot u ^ swz(r) of that row in LDS.  With
    // this XOR swizzle the 16 lanes of a transposed read (4 rows x 32 bytes)
    // hit 8 distinct 16-byte bank groups, without padding the rows.
    auto swz = [](int r) { return (2 * r) & (LPR - 1); };

    // Contiguous caches are read through buffer resources whose range ends at
    // row t_end of this (sequence, KV head): rows past the split read as zeros
    // without touching memory, so no clamping is needed.  Paged caches clamp
    // the row to t_end - 1 (always a valid, finite row of this sequence).
    const size_t rows_bytes = static_cast<size_t>(t_end) * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_uniform_rsrc(kbase + seq_off, static_cast<int>(rows_bytes));
    const __amdgpu_buffer_rsrc_t vrs = make_uniform_rsrc(vbase + seq_off, static_cast<int>(rows_bytes));

    // MODE 2: buffer resource of the 16-row group starting at row0 (wave-
    // uniform, a multiple of 16): its range ends at the last row < t_end, so
    // rows past the split read as zeros without a table lookup or memory access.
    auto group_rsrc = [&](const uint16_t* pool, int row0_) -> __amdgpu_buffer_rsrc_t {
        // wave-uniform by construction; readfirstlane lets the compiler see it
        const int row0 = __builtin_amdgcn_readfirstlane(row0_);
        int nvalid = __builtin_amdgcn_readfirstlane(t_end) - row0;
        nvalid = nvalid < 0 ? 0 : (nvalid > 16 ? 16 : nvalid);
        // (a division leaves its result in a vector register: readfirstlane
        // returns it to a scalar one, so the table read is a scalar load)
        const int lb = __builtin_amdgcn_readfirstlane(row0 / p.block_size);
        const int in_blk = row0 - lb * p.block_size;
        int blk = 0;
        if (nvalid > 0) {
            blk = __builtin_amdgcn_readfirstlane(table[lb]);
            blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
        }
        const uint16_t* g0 = pool + ((static_cast<size_t>(blk) * p.H_kv + j) * p.block_size + in_blk) * D;
        return make_uniform_rsrc(g0, nvalid * D * 2);
    };

    // K rows of a tile, straight into A operands (registers)
    auto load_k = [&](int base, uint4 (&ka)[2][KK]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int t = base + 16 * kb + r16;
            if constexpr (MODE == 2) {
                const __amdgpu_buffer_rsrc_t rs = group_rsrc(kbase, base + 16 * kb);
                const int off = (r16 * D + 8 * q4) * 2;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * kk, 0, 0));
            } else if constexpr (PAGED) {
                const size_t off = row_off(t < t_end ? t : t_end - 1) + 8 * q4;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = *reinterpret_cast<const uint4*>(kbase + off + 32 * kk);
            } else {
                const int off = (t * D + 8 * q4) * 2;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64 * kk, 0, 0));
            }
        }
    };
    // V rows of a tile, HBM -> LDS without passing through registers: lane l
    // of load i fills LDS bytes [16 l, 16 l + 16) of that load's 1 KiB, i.e. row
    // VROWS*i + l / LPR, slot l % LPR, so it fetches chunk (slot ^ swz(row)).
    auto load_v = [&](int base, char* buf) {
        char* wbuf = buf + wave * STAGE;
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int r = VROWS * i + lane / LPR;
            const int u = (lane % LPR) ^ swz(r);
            const int t = base + r;
            lds_void_t* dst = (lds_void_t*)(wbuf + 1024 * i);
            if constexpr (MODE == 2) {
                const int row0 = (VROWS * i / 16) * 16;           // this load's 16-row group
                const __amdgpu_buffer_rsrc_t rs = group_rsrc(vbase, base + row0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ((r - row0) * D + 8 * u) * 2, 0, 0, 0);
            } else if constexpr (PAGED) {
                const uint16_t* src = vbase + row_off(t < t_end ? t : t_end - 1) + 8 * u;
                __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, dst, 16, (t * D + 8 * u) * 2, 0, 0, 0);
            }
        }
    };

    // Plain decode: the first tile's loads go out before the query is loaded,
    // so the two latencies overlap.  The fused step loads the first tile after
    // the query rotation and the append (the split storing the new token may
    // only read it after the store), the same way in every split so that all
    // paths into the pipeline have the same loads in flight.
    uint4 ka0[2][KK], ka1[2][KK];
    constexpr int kStep = NW * TT;
    int base = t_begin + wave * TT;
    if (!FUSED && base < t_end) {
        load_k(base, ka0);
        load_v(base, vbuf0);
    }

    // B operand Q^T: lane holds head 16*hb + r16, d = 32*kk + 8*q4 .. +7
    uint4 qb[HB][KK];
    const int pos = L - 1;                // slot of the new token (fused step)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int g = 16 * hb + r16;
        const size_t qoff = (static_cast<size_t>(b) * p.H_q + j * G + g) * D + 8 * q4;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qb[hb][kk] = make_uint4(0, 0, 0, 0);
            if (g < G)
                qb[hb][kk] = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(FUSED ? p.q_raw : p.q) + qoff + 32 * kk);
        }
        if constexpr (FUSED) {
            // rotate the raw query at the new token's position, exactly as the
            // append kernel would (float32, one rounding per op, then bf16 RNE)
            if (g < G && L > 0) {
                const float* cs = p.rope_cos + static_cast<size_t>(pos) * (D / 2);
                const float* sn = p.rope_sin + static_cast<size_t>(pos) * (D / 2);
                if (p.rope_style == KVC_ROPE_HALF) {
#pragma unroll
                    for (int kk = 0; kk < KK / 2; ++kk) {
                        uint32_t* x = reinterpret_cast<uint32_t*>(&qb[hb][kk]);
                        uint32_t* y = reinterpret_cast<uint32_t*>(&qb[hb][kk + KK / 2]);
                        const int i0 = 32 * kk + 8 * q4;                  // pairs i0 .. i0 + 7
                        float c8[8], s8[8];
                        *reinterpret_cast<float4*>(c8) = *reinterpret_cast<const float4*>(cs + i0);
                        *reinterpret_cast<float4*>(c8 + 4) = *reinterpret_cast<const float4*>(cs + i0 + 4);
                        *reinterpret_cast<float4*>(s8) = *reinterpret_cast<const float4*>(sn + i0);
                        *reinterpret_cast<float4*>(s8 + 4) = *reinterpret_cast<const float4*>(sn + i0 + 4);
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            float a0, a1, b0, b1;
                            rope_pair(bf16_lo(x[w]), bf16_lo(y[w]), c8[2 * w], s8[2 * w], a0, b0);
                            rope_pair(bf16_hi(x[w]), bf16_hi(y[w]), c8[2 * w + 1], s8[2 * w + 1], a1, b1);
                            x[w] = pack_bf16x2(a0, a1);
                            y[w] = pack_bf16x2(b0, b1);
                        }
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) {
                        uint32_t* x = reinterpret_cast<uint32_t*>(&qb[hb][kk]);
                        const int i0 = (32 * kk + 8 * q4) / 2;            // pairs i0 .. i0 + 3
                        const float4 c4 = *reinterpret_cast<const float4*>(cs + i0);
                        const float4 s4 = *reinterpret_cast<const float4*>(sn + i0);
                        const float cw[4] = {c4.x, c4.y, c4.z, c4.w};
                        const float sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            float r0, r1;
                            rope_pair(bf16_lo(x[w]), bf16_hi(x[w]), cw[w], sw[w], r0, r1);
                            x[w] = pack_bf16x2(r0, r1);
                        }
                    }
                }
                if (split == 0 && wave == 0 && p.q_rot_out) {
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.q_rot_out) + qoff + 32 * kk) = qb[hb][kk];
                }
            }
        }
    }

    if constexpr (FUSED) {
        // The split holding the new token stores it (rotated key, raw value)
        // before any of its waves reads the tile that contains it; other
        // splits of the sequence never read that slot.
        if (split == nsp - 1 && L > 0) {
            uint16_t* kdst = nullptr;
            uint16_t* vdst = nullptr;
            if constexpr (PAGED) {
                const int blk = table[pos / p.block_size];      // clamped like every row read
                const int bc = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
                const size_t off = ((static_cast<size_t>(bc) * p.H_kv + j) * p.block_size + pos % p.block_size) * D;
                if (blk == bc) {
                    kdst = static_cast<uint16_t*>(const_cast<void*>(p.k)) + off;
                    vdst = static_cast<uint16_t*>(const_cast<void*>(p.v)) + off;
                }
            } else {
                kdst = static_cast<uint16_t*>(const_cast<void*>(p.k)) + seq_off + static_cast<size_t>(pos) * D;
                vdst = static_cast<uint16_t*>(const_cast<void*>(p.v)) + seq_off + static_cast<size_t>(pos) * D;
            }
            if (kdst && wave == 0) {
                const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (static_cast<size_t>(b) * p.H_kv + j) * D;
                const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (static_cast<size_t>(b) * p.H_kv + j) * D;
                const float* cs = p.rope_cos + static_cast<size_t>(pos) * (D / 2);
                const float* sn = p.rope_sin + static_cast<size_t>(pos) * (D / 2);
                for (int i = lane; i < D / 2; i += 64) {
                    int e0, e1;
                    if (p.rope_style == KVC_ROPE_HALF) { e0 = i; e1 = i + D / 2; }
                    else { e0 = 2 * i; e1 = 2 * i + 1; }
                    float r0, r1;
                    rope_pair(bf16_bits_to_f32(kn[e0]), bf16_bits_to_f32(kn[e1]), cs[i], sn[i], r0, r1);
                    kdst[e0] = f32_to_bf16_rne(r0);
                    kdst[e1] = f32_to_bf16_rne(r1);
                    vdst[2 * i] = vn[2 * i];
                    vdst[2 * i + 1] = vn[2 * i + 1];
                }
            }
            __threadfence_block();
            __syncthreads();
        }
        // Every path (split 0 stores the rotated query, the last split stores
        // the new token) enters the tile pipeline with nothing in flight, so
        // the pipeline's waits stay exact.
        __builtin_amdgcn_s_waitcnt(0);
    }

    // transposed-read source of this lane: row tr_row (+16 for the upper half),
    // columns 16*nb + 4*(s16 % 4) .. +3 = chunk 2*nb + (s16 % 4) / 2, half s16 & 1
    const int s16 = lane & 15;
    const int tr_row = 4 * q4 + s16 / 4;

    auto compute_tile = [&](const uint4 (&ka)[2][KK], const char* buf, int base) {
        const char* wbuf = buf + wave * STAGE;
        // scores S^T = K Q^T, scaled to log2 units; tokens past t_end masked
        float s[HB][8];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) acc = mfma16(ka[kb][kk], qb[hb][kk], acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = base + 16 * kb + 4 * q4 + e;
                    s[hb][4 * kb + e] = t < t_end ? acc[e] * p.scale_log2 : -INFINITY;
                }
            }

        // online softmax per head.  The reference max m is only moved when the
        // tile max exceeds it by more than 2^kLazy (then O and l are rescaled);
        // otherwise p = 2^(s - m) <= 2^kLazy, exact after the final division.
        // P^T goes in as two bf16 B operands, hi + lo = p to ~16 significant bits.
        uint4 ph[HB], pl[HB];
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
                for (int nb = 0; nb < NB; ++nb) o[hb][nb] *= alpha;
            }
            float pr[8], ps = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pr[e] = fast_exp2(s[hb][e] - m[hb]);
                ps += pr[e];
            }
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hi[i] = pack2_bf16(pr[2 * i], pr[2 * i + 1]);
                lo[i] = pack2_bf16(pr[2 * i] - bf16_lo(hi[i]), pr[2 * i + 1] - bf16_hi(hi[i]));
            }
            ph[hb] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            pl[hb] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            l[hb] += ps;
        }

        // O^T += V^T P^T: V^T operands read transposed from LDS
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int u = 2 * nb + (s16 % 4) / 2;
            const int r0 = tr_row, r1 = tr_row + 16;
            const char* a0 = wbuf + r0 * ROWB + 16 * (u ^ swz(r0)) + 8 * (s16 & 1);
            const char* a1 = wbuf + r1 * ROWB + 16 * (u ^ swz(r1)) + 8 * (s16 & 1);
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a0);
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a1);
            uint4 va;
            va.x = __builtin_bit_cast(uint2, lo).x;
            va.y = __builtin_bit_cast(uint2, lo).y;
            va.z = __builtin_bit_cast(uint2, hi).x;
            va.w = __builtin_bit_cast(uint2, hi).y;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                o[hb][nb] = mfma16(va, ph[hb], o[hb][nb]);
                o[hb][nb] = mfma16(va, pl[hb], o[hb][nb]);
            }
        }
    };

    // Software pipeline: while one tile is computed, the next one's K rows
    // (registers) and V rows (the other LDS buffer) are in flight.  The next
    // tile is fetched unconditionally - past the split it reads zeros
    // (contiguous: outside the buffer range, no memory traffic) or the clamped
    // last row (paged) - so every path through the loop has the same loads in
    // flight and the compiler waits only for the tile it is about to use.
    if (base < t_end) {
        if (FUSED) {
            load_k(base, ka0);
            load_v(base, vbuf0);
        }
        for (;;) {
            load_k(base + kStep, ka1);
            load_v(base + kStep, vbuf1);
            compute_tile(ka0, vbuf0, base);
            base += kStep;
            if (base >= t_end) break;
            load_k(base + kStep, ka0);
            load_v(base + kStep, vbuf0);
            compute_tile(ka1, vbuf1, base);
            base += kStep;
            if (base >= t_end) break;
        }
    }

    // ---- merge the waves (LDS reused: all waves are past their loops)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) l[hb] = sum_same_head(l[hb]);
    __syncthreads();
    float* sm_o = reinterpret_cast<float*>(vbuf0);                // [NW][16][D]
    float* sm_m = reinterpret_cast<float*>(vbuf1);                // [NW][16]
    float* sm_l = sm_m + NW * 16;                                   // [NW][16]
    const int NT = NW * 64;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int g = 16 * hb + r16;          // this lane's head
        // lane holds O^T[c][g] for c = 16*nb + 4*q4 + e
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm_o[(wave * 16 + r16) * D + 16 * nb + 4 * q4 + e] = o[hb][nb][e];
        if (q4 == 0) {
            sm_m[wave * 16 + r16] = m[hb];
            sm_l[wave * 16 + r16] = l[hb];
        }
        __syncthreads();
        const int heads = min(16, G - 16 * hb);
        for (int idx = tid; idx < heads * D; idx += NT) {
            const int gh = idx / D;
            const int c = idx % D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * 16 + gh]);
            float A = 0.0f, Ls = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = sm_m[w * 16 + gh];
                const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
                A = fmaf(sm_o[(w * 16 + gh) * D + c], f, A);
                Ls = fmaf(sm_l[w * 16 + gh], f, Ls);
            }
            const size_t bh = static_cast<size_t>(b) * p.H_q + j * G + 16 * hb + gh;
            if (nsp == 1) {
                static_cast<uint16_t*>(p.out)[bh * D + c] = f32_to_bf16_rne(Ls > 0.0f ? A / Ls : 0.0f);
            } else {
                p.ws_part[(bh * p.n_splits + split) * D + c] = A;
                if (c == 0) p.ws_ml[bh * p.n_splits + split] = make_float2(M, Ls);
            }
        }
        (void)g;
        __syncthreads();
    }
}

constexpr int kNWm = 4;

template <int D, int HB, bool FUSED>
hipError_t launch_dhf(bool paged, const DecodeParams& p, hipStream_t stream, const KernelTiming& tm) {
    const dim3 grid(p.n_wg_pad), block(kNWm * 64);
    const int32_t* tbl = p.block_table;
    if (!paged) return launch_timed(decode_mfma_kernel<D, HB, kNWm, 0, FUSED>, grid, block, stream, tm, p, tbl);
    if (p.block_size % 16 == 0 && p.split_tokens % 32 == 0)
        return launch_timed(decode_mfma_kernel<D, HB, kNWm, 2, FUSED>, grid, block, stream, tm, p, tbl);
    return launch_timed(decode_mfma_kernel<D, HB, kNWm, 1, FUSED>, grid, block, stream, tm, p, tbl);
}

template <int D>
hipError_t launch_d(int G, bool paged, bool fused, const DecodeParams& p, hipStream_t stream,
                    const KernelTiming& tm) {
    if (G <= 16)
        return fused ? launch_dhf<D, 1, true>(paged, p, stream, tm) : launch_dhf<D, 1, false>(paged, p, stream, tm);
    return fused ? launch_dhf<D, 2, true>(paged, p, stream, tm) : launch_dhf<D, 2, false>(paged, p, stream, tm);
}

}  // namespace

bool decode_mfma_supported(kvc_dtype dtype, int d, int G) {
    return dtype == KVC_BF16 && (d == 64 || d == 128 || d == 256) && G >= 1 && G <= 32;
}

int decode_mfma_tile_tokens() { return 32 * kNWm; }

hipError_t launch_decode_mfma(int d, int G, bool paged, bool fused, const DecodeParams& p,
                              hipStream_t stream, const KernelTiming& tm) {
    switch (d) {
        case 64: return launch_d<64>(G, paged, fused, p, stream, tm);
        case 128: return launch_d<128>(G, paged, fused, p, stream, tm);
        case 256: return launch_d<256>(G, paged, fused, p, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
