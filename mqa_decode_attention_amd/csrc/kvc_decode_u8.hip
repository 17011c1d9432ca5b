// kvc_decode_u8.hip - decode attention over an 8-bit KV cache (uint8 codes on
// an affine grid, or FP8 E4M3 / E5M2 codes with a scale) on the gfx950 matrix
// cores.
//
// FP8 caches (FMT kQ8E4M3 / kQ8E5M2; the one-byte FP8 caches of "Arsitektur
// Inferensi LLM", tveniu.com, sections 2 and 8): each vector's codes with a
// (scale, 0) pair, reading back as decode(code) * scale.  Every E4M3 or E5M2
// value is exact in bf16, so they enter the products as the uint8 codes do,
// and a zero point of 0 makes the corrections below vanish.
//
// Cache: each cached key or value vector is d uint8 codes c plus one float
// (step, zero point) pair, and reads back as (c - zp) * step - the
// QuantizedKVCache listing of "KV Cache 최적화 심층 분석: GQA·MLA·MHA 어텐션
// 메커니즘과 메모리 효율화 전략" (youngju.dev), with a pair kept per vector.
// Attention is the unquantized one ("Grouped-query attention: berbagi KV head di
// antara grup query", nalar.dev, section "Jumlah head menentukan batas grup")
// over those values.  The affine map stays out of the two products: the codes
// are exact in bf16, and
//     q . k_t          = step_t * (q . c_t - zp_t * sum(q))
//     sum_t p_t v_t[c] = sum_t (p_t * step_t) c_t[c] - sum_t p_t * step_t * zp_t
// so both MFMA products take the raw codes; each score gets one multiply-add,
// each weight one multiply, and each head one running correction that is
// subtracted from O at the end.
//
// Structure (as the bf16 kernel's staged-tile path): one workgroup of four
// waves per (sequence, KV head, split); each wave streams 32-token tiles.  Per
// tile the K codes and V codes go from HBM to LDS by direct loads (buffer
// ranges ending at the split, so nothing past it is read), the pair rows with
// them (paged) or four tiles' at a time in one load (contiguous); the K
// operand is read from LDS as 8 codes per lane and converted to bf16; the V
// operand V^T is read from the staged codes transposed (ds_read_b64_tr_b8:
// each lane gets one column's codes of 8 token rows) and converted the same
// way.  Each stage is refilled as soon as the tile is done with it (K after
// its operand reads, V after its transposed reads), after every LDS read of it
// has completed.  MODE 0: contiguous codes [B, H_kv, T_max, d], pairs
// [B, H_kv, T_max, 2].  MODE 3: pools [N_blk, H_kv, bs, d] / [.., bs, 2] with
// bs % 16 == 0; the split's slice of the block table is staged in LDS.
//
// Fused step (FUSED): the append runs inside the streaming pass, as in the
// bf16 kernel.  Every workgroup rotates its queries in registers; the last
// split of a (sequence, KV head) also rotates the new key (float32, not
// rounded), quantizes it and the raw new value exactly as the append kernel
// does (min and max over the vector, step = (max - min) / 255, zero point and
// codes rounded to nearest even and clamped to [0, 255]), patches the codes
// and pairs into the tile it loaded (the stored row may not have landed yet)
// and stores them once all its loads are done.

#include <type_traits>

#include "kvc_internal.h"
#include "kvc_device.h"
#include "kvc_mfma_common.h"

namespace kvc {

namespace {

using namespace mfma;

constexpr int kNWq = 4;      // waves per workgroup
constexpr int kTTq = 32;     // tokens per wave tile
constexpr int kGrpq = 4;     // contiguous caches: tiles whose pair rows come in one load

// Eight codes -> eight bf16 values, exact.  uint8 codes: integers below 256
// need 8 significant bits; each byte converted to float32
// (v_cvt_f32_ubyteN).  FP8 codes: at most 4 significant bits and exponents
// well inside bf16's range; two codes per conversion (v_cvt_pk_f32_fp8 for
// E4M3, v_cvt_pk_f32_bf8 for E5M2, reading the OCP formats on gfx950).  The
// bf16 values are the float32 results' upper halves.
__device__ __forceinline__ float byte_f32(uint32_t w, int k) { return static_cast<float>((w >> (8 * k)) & 0xFFu); }
__device__ __forceinline__ uint32_t hi_halves(float hi, float lo) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}
template <int FMT>
__device__ __forceinline__ uint4 codes8_to_bf16(uint2 c) {
    uint4 r;
    if constexpr (FMT == kQ8Affine) {
        const float f0 = byte_f32(c.x, 0), f1 = byte_f32(c.x, 1), f2 = byte_f32(c.x, 2), f3 = byte_f32(c.x, 3);
        const float f4 = byte_f32(c.y, 0), f5 = byte_f32(c.y, 1), f6 = byte_f32(c.y, 2), f7 = byte_f32(c.y, 3);
        r.x = hi_halves(f1, f0);
        r.y = hi_halves(f3, f2);
        r.z = hi_halves(f5, f4);
        r.w = hi_halves(f7, f6);
    } else {
        // (the word select is an immediate)
#define KVC_CVT_PK(w, upper) (FMT == kQ8E4M3 ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), upper) \
                                             : __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), upper))
        const auto a = KVC_CVT_PK(c.x, false), b = KVC_CVT_PK(c.x, true);
        const auto e = KVC_CVT_PK(c.y, false), f = KVC_CVT_PK(c.y, true);
#undef KVC_CVT_PK
        r.x = hi_halves(a[1], a[0]);
        r.y = hi_halves(b[1], b[0]);
        r.z = hi_halves(e[1], e[0]);
        r.w = hi_halves(f[1], f[0]);
    }
    return r;
}

// Slot of the 16-byte chunk u of staged V code row r (an XOR swizzle; also
// the chunk held by slot u).  A 64-bit LDS read is served 32 lanes (256
// bytes, one sweep of the banks) at a time; in a transposed read those lanes
// take one chunk of the 16 rows 8 h + 0..7 and 16 + 8 h + 0..7 (h = 0, 1),
// and the swizzle gives the rows that share banks distinct slots (d = 128:
// rows of equal parity; d = 64: rows equal mod 4).
template <int D>
__device__ __forceinline__ int vslot(int r, int u) {
    if constexpr (D == 128) return u ^ (((r >> 1) & 3) | (((r >> 4) & 1) << 2));
    else return u ^ (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}

// (one 16-head block: registers held to two waves per SIMD, so that two
// workgroups share a CU as planned)
template <int D, int HB, int MODE, bool FUSED, bool BAL, int FMT>
__global__ void __launch_bounds__(kNWq * 64) __attribute__((amdgpu_waves_per_eu(HB == 1 ? 2 : 1, 8)))
decode_u8_kernel(const DecodeParams p, const int32_t* __restrict__ block_table, float* k_sz, float* v_sz) {
    constexpr bool PAGED = MODE == 3;
    constexpr int NW = kNWq;
    constexpr int TT = kTTq;
    constexpr int KB = TT / 16;           // 16-row blocks per tile
    constexpr int KK = D / 32;            // 32-wide d slices of the score product
    constexpr int NB = D / 16;            // 16-column blocks of V
    constexpr int CROW = D;               // bytes per code row
    constexpr int CLPR = D / 16;          // 16-byte chunks per code row
    constexpr int CROWS = 64 / CLPR;      // code rows per wave-wide 16-byte load
    constexpr int CLOADS = TT / CROWS;    // such loads per tile and tensor
    constexpr int CSTAGE = TT * CROW;     // LDS bytes of one code tile
    // pair rows: 32 tokens x 8 bytes, one load (contiguous) or one per 16-row
    // block (paged: the halves may lie in different blocks)
    constexpr int SZLOADS = PAGED ? 2 : 1;
    constexpr int SZROWS = TT / SZLOADS;  // rows per pair load
    static_assert(CROWS <= 16 && TT % CROWS == 0, "code rows per load");

    // the K and V code stages (one array: the epilogue reuses it whole)
    __shared__ __attribute__((aligned(16))) char code_lds[2 * NW * CSTAGE];
    char* const kc_lds = code_lds;
    char* const vc_lds = code_lds + NW * CSTAGE;
    // pair rows per wave and tensor: paged, one tile's; contiguous (GP), two
    // buffers of kGrp tiles' rows, a group's rows requested in one load
    constexpr bool GP = !PAGED;
    constexpr int kGrp = kGrpq;
    constexpr int PBYTES = GP ? 2 * kGrp * TT * 8 : TT * 8;
    __shared__ __attribute__((aligned(16))) char ksz_lds[NW * PBYTES];
    __shared__ __attribute__((aligned(16))) char vsz_lds[NW * PBYTES];
    __shared__ int tbl_lds[PAGED ? kTblMax : 1];
    __shared__ int s_last;                 // the in-kernel merge: this workgroup arrived last
    __shared__ std::conditional_t<BAL, BalLds, char> bal;   // the balanced schedule's lengths and prefix
    static_assert(NW * TT * 8 >= 2 * NW * 16 * 4, "merge area");
    static_assert(!BAL || PAGED, "the balanced schedule serves paged pools");
    constexpr int kStep = NW * TT;        // tokens per loop step of the workgroup

    const int wid = blockIdx.x < static_cast<unsigned>(p.n_wg) ? static_cast<int>(blockIdx.x) : -1;
    if (wid < 0) return;

    // Balanced schedule (paged pools with ragged lengths; the helpers in
    // kvc_mfma_common.h): every workgroup reads all lengths, then runs its
    // split body once per segment of its equal share of all units' steps.
    if constexpr (BAL) {
        if (!bal_setup<NW * 64, kStep, FUSED>(p, wid, bal)) return;
    }

    // (one pass under the split schedule: a trip count the compiler can see
    // keeps its register allocation that of straight-line code)
    for (int it = 0; BAL || it < 1; ++it) {
    // ---- one split (balanced schedule: one segment) of one unit
    int unit, split, nsp, t_begin, t_end, L, pos;
    BalSeg sg{};
    if constexpr (BAL) {
        if (!bal_segment<kStep, FUSED>(p, wid, it, bal, sg)) break;
        unit = sg.unit;
        nsp = sg.nsp;
        split = sg.split;
        L = sg.L;
        pos = sg.pos;
        t_begin = sg.t_begin;
        t_end = sg.t_end;
        // (the previous segment's output stores, before this one's loads)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
        split = wid % p.n_splits;
        unit = wid / p.n_splits;          // b * H_kv + j
        // (the quantized entry points have no window: the range is [0, L))
        pos = FUSED ? p.positions[unit / p.H_kv] : 0;
        L = FUSED ? len_from_position(p, pos) : attended_len(p, unit / p.H_kv);
        nsp = (L + p.split_tokens - 1) / p.split_tokens;
        nsp = nsp < 1 ? 1 : nsp;
        if (split >= nsp) return;
        t_begin = split * p.split_tokens;
        t_end = min(L, t_begin + p.split_tokens);
    }
    const int b = unit / p.H_kv;
    const int j = unit % p.H_kv;
    const int G = p.G;

    // (the lane index opaque to the compiler inside each segment of the
    // balanced schedule, so the per-lane offsets derived from it are not
    // hoisted above the segment loop and kept live through every epilogue)
    int tid = threadIdx.x;
    if constexpr (BAL) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int q4 = lane >> 4;

    float m[HB], l[HB], corr[HB];
    f32x4_t o[HB][NB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        m[hb] = -kNoMax;
        l[hb] = 0.0f;
        corr[hb] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[hb][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const uint8_t* kcodes = static_cast<const uint8_t*>(p.k);
    const uint8_t* vcodes = static_cast<const uint8_t*>(p.v);
    const size_t seq_rows = PAGED ? 0 : (static_cast<size_t>(b) * p.H_kv + j) * p.T_max;
    const int32_t* table = PAGED ? block_table + static_cast<size_t>(b) * p.max_blocks_per_seq : nullptr;
    const int fb = PAGED ? t_begin / p.block_size : 0;

    // buffer resource of rows [row0, row0 + n) of one vector array (codes of
    // `width` bytes per row, or pairs of 8), its range cut at t_end: rows past
    // the split read as zeros without a memory access.  Contiguous: rows of
    // this (sequence, KV head); paged: the 16-row group at row0 (a multiple
    // of 16) lies in one block, found in the staged table.
    // (blk_: the group's block id from the staged table, read by the caller)
    auto rows_rsrc = [&](const void* base_ptr, int width, int row0_, int n, int blk_) -> __amdgpu_buffer_rsrc_t {
        const int row0 = __builtin_amdgcn_readfirstlane(row0_);
        int nvalid = __builtin_amdgcn_readfirstlane(t_end) - row0;
        nvalid = nvalid < 0 ? 0 : (nvalid > n ? n : nvalid);
        size_t first;
        if constexpr (PAGED) {
            const int lb = row0 / p.block_size;
            const int blk = __builtin_amdgcn_readfirstlane(nvalid > 0 ? blk_ : 0);
            first = (static_cast<size_t>(blk) * p.H_kv + j) * p.block_size + (row0 - lb * p.block_size);
        } else {
            first = seq_rows + static_cast<size_t>(row0);
        }
        return make_uniform_rsrc(static_cast<const char*>(base_ptr) + first * width, nvalid * width);
    };

    // one tensor's tile at row base: codes (CLOADS loads) then pairs (SZLOADS)
    // into this wave's LDS slices.  Codes: lane l of load i fills bytes
    // [16 l, 16 l + 16) of that load's 1 KiB, i.e. row CROWS*i + l / CLPR,
    // slot l % CLPR; K rows hold chunk (slot ^ ((row / (256 / CROW)) % CLPR))
    // there (the 32 lanes reading one chunk of 16 rows for the operand, 256
    // bytes, then cover every bank once), V rows chunk vslot(row, slot).
    // Block ids of the two 16-row groups of the tile at row base (paged):
    // read once per tile, unconditionally (index clamped into the slice;
    // groups past the split get a zero range whatever they read), and shared
    // by its code and pair loads.  Read per load instead, each load waited
    // for its own table read.
    struct TileBlocks {
        int g[2];
    };
    auto tile_blocks = [&](int base) __attribute__((always_inline)) {
        TileBlocks tb{};
        if constexpr (PAGED) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                int ti = __builtin_amdgcn_readfirstlane(base + 16 * g) / p.block_size - fb;
                ti = ti < 0 ? 0 : (ti >= kTblMax ? kTblMax - 1 : ti);
                tb.g[g] = tbl_lds[ti];
            }
        }
        return tb;
    };
    auto load_tensor = [&](auto is_k, int base, const TileBlocks& tb) __attribute__((always_inline)) {
        constexpr bool ISK = decltype(is_k)::value;
        const uint8_t* codes = ISK ? kcodes : vcodes;
        const float* sz = ISK ? k_sz : v_sz;
        char* cbuf = (ISK ? kc_lds : vc_lds) + wave * CSTAGE;
        char* sbuf = (ISK ? ksz_lds : vsz_lds) + wave * PBYTES;
#pragma unroll
        for (int i = 0; i < CLOADS; ++i) {
            const int r = CROWS * i + lane / CLPR;
            const int u = ISK ? ((lane % CLPR) ^ ((r / (256 / CROW)) % CLPR)) : vslot<D>(r, lane % CLPR);
            const int g0 = (CROWS * i / 16) * 16;                 // this load's 16-row group
            const __amdgpu_buffer_rsrc_t rs =
                rows_rsrc(codes, CROW, base + (PAGED ? g0 : 0), PAGED ? 16 : TT, tb.g[g0 / 16]);
            const int row_in = PAGED ? r - g0 : r;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(cbuf + 1024 * i), 16,
                                                     row_in * CROW + 16 * u, 0, 0, kNT);
        }
        if constexpr (GP) return;          // (pair rows by group: load_pair_group)
#pragma unroll
        for (int i = 0; i < SZLOADS; ++i) {
            // SZROWS rows of 8 bytes are SZROWS / 2 lanes of 16 bytes; the other
            // lanes stay idle, so the load writes only those bytes of LDS (the
            // instruction is still issued once per wave: the wait counts hold)
            const __amdgpu_buffer_rsrc_t rs = rows_rsrc(sz, 8, base + SZROWS * i, SZROWS, tb.g[PAGED ? i : 0]);
            if (lane < SZROWS / 2)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(sbuf + 8 * SZROWS * i), 16, 16 * lane, 0,
                                                         0, kNT);
        }
    };
    constexpr int kTensorLoads = CLOADS + SZLOADS;
    // (GP) the pair rows of the wave's kGrp tiles from row gbase on (strided
    // by kStep) into group buffer gb: lanes 16 k .. 16 k + 15 take tile k's
    // TT rows, 16 bytes each; the range ends at t_end as for every tile.
    auto load_pair_group = [&](auto is_k, int gbase, int gb) __attribute__((always_inline)) {
        constexpr bool ISK = decltype(is_k)::value;
        static_assert(kGrp * TT * 8 == 64 * 16, "one 16-byte piece per lane");
        const float* sz = ISK ? k_sz : v_sz;
        char* sbuf = (ISK ? ksz_lds : vsz_lds) + wave * PBYTES + gb * kGrp * TT * 8;
        const __amdgpu_buffer_rsrc_t rs = rows_rsrc(sz, 8, gbase, (kGrp - 1) * kStep + TT, 0);
        const int k = lane / 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)sbuf, 16, (k * kStep + 2 * (lane % 16)) * 8, 0, 0,
                                                 kNT);
    };


    // Prologue: the table slice (paged), then the query, then the first tile.
    int base = t_begin + wave * TT;
    constexpr int kTblPer = kTblMax / (NW * 64);
    int tv[kTblPer];
    const int nblk = PAGED ? (t_end - 1) / p.block_size - fb + 1 : 0;
    if constexpr (PAGED) {
#pragma unroll
        for (int k = 0; k < kTblPer; ++k) {
            const int i = tid + k * NW * 64;
            tv[k] = table[fb + (i < nblk ? i : 0)];
        }
    }
    const size_t qgrp = (static_cast<size_t>(b) * p.H_q + static_cast<size_t>(j) * G) * D;
    const __amdgpu_buffer_rsrc_t qrs =
        make_uniform_rsrc(static_cast<const uint16_t*>(FUSED ? p.q_raw : p.q) + qgrp, G * D * 2);
    uint4 qb[HB][KK];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qb[hb][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                qrs, ((16 * hb + r16) * D + 32 * kk + 8 * q4) * 2, 0, 0));

    // Fused step: the new key and value in the operand layout (lane (r16, q4)
    // holds elements 32 kk + 8 q4 .. +7 of chunk kk; the last split only -
    // other workgroups get a zero range) and the rotation row of the slot.
    const bool pos_ok = FUSED && pos >= 0 && pos < p.capacity && pos < p.rope_rows;
    const bool own = pos_ok && split == nsp - 1;
    const bool half = FUSED && p.rope_style == KVC_ROPE_HALF;
    uint4 kraw[FUSED ? KK : 1], vraw[FUSED ? KK : 1];
    float4 cw[FUSED ? KK : 1], sw[FUSED ? KK : 1];
    if constexpr (FUSED) {
        const size_t kv_in = (static_cast<size_t>(b) * p.H_kv + j) * D;
        const __amdgpu_buffer_rsrc_t knrs =
            make_uniform_rsrc(static_cast<const uint16_t*>(p.k_new) + kv_in, own ? D * 2 : 0);
        const __amdgpu_buffer_rsrc_t vnrs =
            make_uniform_rsrc(static_cast<const uint16_t*>(p.v_new) + kv_in, own ? D * 2 : 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            kraw[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(knrs, (32 * kk + 8 * q4) * 2, 0, 0));
            vraw[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vnrs, (32 * kk + 8 * q4) * 2, 0, 0));
        }
        // interleaved pairs: chunk kk holds pairs 16 kk + 4 q4 .. +3; split
        // halves: chunks m and m + KK/2 pair element by element, pairs
        // 32 m + 8 q4 .. +7, as cw[2m], cw[2m + 1]  (row 0 stands in for an
        // invalid position: nothing is then rotated or stored)
        const size_t trow = static_cast<size_t>(pos_ok ? pos : 0) * (D / 2);
        const __amdgpu_buffer_rsrc_t crs = make_uniform_rsrc(p.rope_cos + trow, D * 2);
        const __amdgpu_buffer_rsrc_t srs = make_uniform_rsrc(p.rope_sin + trow, D * 2);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int i0 = half ? 32 * (kk >> 1) + 8 * q4 + 4 * (kk & 1) : 16 * kk + 4 * q4;
            cw[kk] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(crs, i0 * 4, 0, 0));
            sw[kk] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(srs, i0 * 4, 0, 0));
        }
    }
    if constexpr (PAGED) {
#pragma unroll
        for (int k = 0; k < kTblPer; ++k) {
            const int i = tid + k * NW * 64;
            const int blk = tv[k] < 0 ? 0 : (tv[k] >= p.num_blocks ? p.num_blocks - 1 : tv[k]);
            if (i < nblk) tbl_lds[i] = blk;
        }
        __syncthreads();
    }
    {
        const TileBlocks tb0 = tile_blocks(base);
        if constexpr (GP) {
            load_pair_group(std::true_type{}, base, 0);
            load_pair_group(std::false_type{}, base, 0);
        }
        load_tensor(std::true_type{}, base, tb0);
        load_tensor(std::false_type{}, base, tb0);
    }

    // Fused step: rotate the queries (bf16, as stored by the append) and the
    // new key (float32), quantize the key and the value.
    uint2 kcode[FUSED ? KK : 1] = {}, vcode[FUSED ? KK : 1] = {};   // 8 codes per chunk
    float2 kpair = make_float2(0.0f, 0.0f), vpair = make_float2(0.0f, 0.0f);
    int patch_row = -1;                   // token index of the patched row, or -1
    size_t slot_row = 0;                  // vector index of the new token's slot
    bool slot_ok = false;
    if constexpr (FUSED) {
        auto fget = [](const float4& v, int i) __attribute__((always_inline)) {
            return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
        };
        // one vector in the operand layout -> rotated float32 values
        auto rotate = [&](const uint4 (&x)[KK], float (&r)[KK][8]) __attribute__((always_inline)) {
            if (half) {
#pragma unroll
                for (int m = 0; m < KK / 2; ++m) {
                    const uint32_t* xa = reinterpret_cast<const uint32_t*>(&x[m]);
                    const uint32_t* ya = reinterpret_cast<const uint32_t*>(&x[m + KK / 2]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float a = (e & 1) ? bf16_hi(xa[e / 2]) : bf16_lo(xa[e / 2]);
                        const float c = (e & 1) ? bf16_hi(ya[e / 2]) : bf16_lo(ya[e / 2]);
                        rope_pair(a, c, fget(cw[2 * m + e / 4], e % 4), fget(sw[2 * m + e / 4], e % 4), r[m][e],
                                  r[m + KK / 2][e]);
                    }
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const uint32_t* xa = reinterpret_cast<const uint32_t*>(&x[kk]);
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        rope_pair(bf16_lo(xa[w]), bf16_hi(xa[w]), fget(cw[kk], w), fget(sw[kk], w), r[kk][2 * w],
                                  r[kk][2 * w + 1]);
                }
            }
        };
        if (pos_ok) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                float r[KK][8];
                rotate(qb[hb], r);
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    qb[hb][kk] = make_uint4(pack_bf16x2(r[kk][0], r[kk][1]), pack_bf16x2(r[kk][2], r[kk][3]),
                                            pack_bf16x2(r[kk][4], r[kk][5]), pack_bf16x2(r[kk][6], r[kk][7]));
            }
        }
        // quantize one vector (the four lanes q4 = 0..3 of a row hold all of
        // it): the affine grid of its min and max, codes rounded and clamped;
        // FP8: the scale of its largest magnitude (E4M3) or 1 (E5M2), codes
        // of x / scale rounded to nearest even and saturated, as the append
        // kernel does
        auto quantize = [&](const float (&x)[KK][8], uint2 (&code)[KK], float2& pair) __attribute__((always_inline)) {
            if constexpr (FMT != kQ8Affine) {
                float scale = 1.0f;
                if constexpr (FMT == kQ8E4M3) {
                    float amax = 0.0f;
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[kk][e]));
                    amax = max_same_head(amax);
                    scale = amax / 448.0f;
                    scale = scale == 0.0f ? 1.0f : scale;
                }
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    uint32_t w[2] = {0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e / 4] |= fp8_encode<FMT>(x[kk][e] / scale) << (8 * (e % 4));
                    code[kk] = make_uint2(w[0], w[1]);
                }
                pair = make_float2(scale, 0.0f);
                return;
            }
            float mn = x[0][0], mx = x[0][0];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    mn = fminf(mn, x[kk][e]);
                    mx = fmaxf(mx, x[kk][e]);
                }
            mn = fminf(mn, __shfl_xor(mn, 16, 64));
            mn = fminf(mn, __shfl_xor(mn, 32, 64));
            mx = max_same_head(mx);
            float step = (mx - mn) / 255.0f;
            step = step == 0.0f ? 1.0f : step;
            const float zp = fminf(fmaxf(rintf(-mn / step), 0.0f), 255.0f);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                uint32_t w[2] = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t c = static_cast<uint32_t>(fminf(fmaxf(rintf(x[kk][e] / step + zp), 0.0f), 255.0f));
                    w[e / 4] |= c << (8 * (e % 4));
                }
                code[kk] = make_uint2(w[0], w[1]);
            }
            pair = make_float2(step, zp);
        };
        // (only the split that stores the token: the divisions of the
        // quantizer would delay every other workgroup's first tile)
        if (own) {
            float kf[KK][8], vf[KK][8];
            rotate(kraw, kf);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint32_t* xa = reinterpret_cast<const uint32_t*>(&vraw[kk]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    vf[kk][2 * w] = bf16_lo(xa[w]);
                    vf[kk][2 * w + 1] = bf16_hi(xa[w]);
                }
            }
            quantize(kf, kcode, kpair);
            quantize(vf, vcode, vpair);
        }

        // the new token's slot (a clamped table entry would be another
        // sequence's block: then nothing is stored)
        if constexpr (PAGED) {
            if (own) {
                const int blk = table[pos / p.block_size];
                slot_ok = blk >= 0 && blk < p.num_blocks;
                slot_row = (static_cast<size_t>(slot_ok ? blk : 0) * p.H_kv + j) * p.block_size + pos % p.block_size;
            }
        } else {
            slot_ok = own;
            slot_row = seq_rows + static_cast<size_t>(own ? pos : 0);
        }
        patch_row = __builtin_amdgcn_readfirstlane(slot_ok && pos < t_end ? pos : -1);
    }

    // sum over d of each query head (the zero-point term of the scores): this
    // lane's 8*KK elements, then the four lanes of the head.  FP8 caches read
    // back as decode(code) * scale: no zero-point terms at all (ZP false).
    constexpr bool ZP = FMT == kQ8Affine;
    float qsum[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        if constexpr (!ZP) {
            qsum[hb] = 0.0f;
            continue;
        }
        float acc = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(&qb[hb][kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += bf16_lo(w[i]) + bf16_hi(w[i]);
        }
        qsum[hb] = sum_same_head(acc);
    }

    const int s16 = lane & 15;

    // One tile.  GP: phase = the tile's place in its group, gsel = the
    // group's pair buffer.  A wave's loads go out in this order: the
    // prologue's K and V pair groups 0, K codes 0, V codes 0; then in each
    // tile the next tile's K codes after its K reads and V codes after its V
    // reads, and at phase 0 after those the next K and V pair groups.  A
    // tile's pair group is older than its codes, and waiting for its K or V
    // codes leaves CLOADS later loads outstanding (at phase 1 it could leave
    // CLOADS + 2: there it also waits for two loads of the previous tile).
    // Paged: codes and pairs per tile, kTensorLoads per tensor.
    auto compute_tile = [&](int base, int phase, int gsel) __attribute__((always_inline)) {
        const char* kc = kc_lds + wave * CSTAGE;
        const char* vc = vc_lds + wave * CSTAGE;
        const int poff = GP ? wave * PBYTES + (gsel * kGrp + phase) * TT * 8 : wave * TT * 8;
        char* ks = ksz_lds + poff;
        char* vs = vsz_lds + poff;
        // block ids of the next tile (paged), before the waits below cover them
        const TileBlocks tb_next = tile_blocks(base + kStep);

        constexpr int kWait = GP ? CLOADS : kTensorLoads;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait));
        // fused step: the tile holding the new token gets its codes and pair
        // over what was loaded for that row (every read below comes after)
        const int dp = patch_row - base;
        const bool patch = FUSED && static_cast<unsigned>(dp) < static_cast<unsigned>(TT);
        if constexpr (FUSED) {
            if (patch) {
                char* kcw = kc_lds + wave * CSTAGE;
                if (r16 == 0) {
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) {
                        const int c8 = 4 * kk + q4;
                        *reinterpret_cast<uint2*>(kcw + dp * CROW + 16 * ((c8 / 2) ^ ((dp / (256 / CROW)) % CLPR)) + 8 * (c8 % 2)) =
                            kcode[kk];
                    }
                }
                if (lane == 0) *reinterpret_cast<float2*>(ks + 8 * dp) = kpair;
            }
        }
        // The K operand's codes and the K pairs, read as inline assembly for
        // the reason given at the V^T reads below (through plain loads they
        // drew a wait for every load in flight, this tile's V included); the
        // wait above is the one they need, and the one below, tied to every
        // result, keeps their uses after the data.
        // (a lane's four pair rows of a 16-row block are 32 contiguous bytes:
        // two 128-bit reads)
        static_assert(KB == 2 && KB * KK + 2 * KB <= 16, "the wait below names every result");
        u32x2_t kw[KB * KK];
        u32x4_t pw4[2 * KB];
        const unsigned kcb = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void_t*)kc));
        const unsigned ksb = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void_t*)ks));
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int r = 16 * kb + r16;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int c8 = 4 * kk + q4;                         // 8-byte piece of the row
                const unsigned a = kcb + r * CROW + 16 * ((c8 / 2) ^ ((r / (256 / CROW)) % CLPR)) + 8 * (c8 % 2);
                asm volatile("ds_read_b64 %0, %1" : "=v"(kw[kb * KK + kk]) : "v"(a) : "memory");
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const unsigned a = ksb + 8 * (16 * kb + 4 * q4) + 16 * h;
                asm volatile("ds_read_b128 %0, %1" : "=v"(pw4[2 * kb + h]) : "v"(a) : "memory");
            }
        }
        if constexpr (KK == 4) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(kw[0]), "+v"(kw[1]), "+v"(kw[2]), "+v"(kw[3]), "+v"(kw[4]), "+v"(kw[5]),
                           "+v"(kw[6]), "+v"(kw[7]), "+v"(pw4[0]), "+v"(pw4[1]), "+v"(pw4[2]), "+v"(pw4[3])
                         :
                         : "memory");
        } else {
            static_assert(KK == 2, "head_dim 64 or 128");
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(kw[0]), "+v"(kw[1]), "+v"(kw[2]), "+v"(kw[3]), "+v"(pw4[0]), "+v"(pw4[1]),
                           "+v"(pw4[2]), "+v"(pw4[3])
                         :
                         : "memory");
        }
        uint4 ka[KB][KK];
        float2 kp[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) ka[kb][kk] = codes8_to_bf16<FMT>(__builtin_bit_cast(uint2, kw[kb * KK + kk]));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 w = __builtin_bit_cast(uint4, pw4[2 * kb + h]);
                kp[kb][2 * h] = make_float2(__builtin_bit_cast(float, w.x), __builtin_bit_cast(float, w.y));
                kp[kb][2 * h + 1] = make_float2(__builtin_bit_cast(float, w.z), __builtin_bit_cast(float, w.w));
            }
        }
        // the K stage is free once those reads are done: the next tile's K
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        load_tensor(std::true_type{}, base + kStep, tb_next);

        // scores: step * (q . c - zp * sum(q)), in log2 units; past t_end masked
        constexpr int NS = 4 * KB;
        float s[HB][NS];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) acc = mfma16(ka[kb][kk], qb[hb][kk], acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float2 sz = kp[kb][e];
                    s[hb][4 * kb + e] = ZP ? (acc[e] - sz.y * qsum[hb]) * (sz.x * p.scale_log2)
                                           : acc[e] * (sz.x * p.scale_log2);
                }
            }
        // (only a tile that reaches past the split has rows to mask)
        if (base + TT > t_end) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int i = 0; i < NS; ++i)
                    if (base + 16 * (i / 4) + 4 * q4 + i % 4 >= t_end) s[hb][i] = -INFINITY;
        }

        // this tile's V codes (and paged, pairs): issued before the K loads
        // just above
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait));
        if constexpr (FUSED) {
            if (patch) {
                char* vcw = vc_lds + wave * CSTAGE;
                if (r16 == 0) {
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) {
                        const int c8 = 4 * kk + q4;
                        *reinterpret_cast<uint2*>(vcw + dp * CROW + 16 * vslot<D>(dp, c8 / 2) + 8 * (c8 % 2)) =
                            vcode[kk];
                    }
                }
                if (lane == 0) *reinterpret_cast<float2*>(vs + 8 * dp) = vpair;
            }
        }
        // the V pairs and this lane's part of the V^T operand: for each
        // 16-column block nb, the codes of column 16 nb + s16 in the 8 token
        // rows whose weights this lane holds (4 q4 + 0..3, 16 + 4 q4 + 0..3),
        // by one transposed read in which lanes 2i and 2i + 1 of each 16 name
        // the two 8-byte halves of row i's chunk nb (inline assembly, as the K
        // reads above; the wait above is the one they need)
        static_assert(2 * KB + NB <= 16, "the wait below names every result");
        u32x4_t vpw[2 * KB];
        u32x2_t vt[NB];
        {
            const unsigned vsb = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void_t*)vs));
            const unsigned vcb = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void_t*)vc));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const unsigned a = vsb + 8 * (16 * kb + 4 * q4) + 16 * h;
                    asm volatile("ds_read_b128 %0, %1" : "=v"(vpw[2 * kb + h]) : "v"(a) : "memory");
                }
            const int ti = s16 >> 1;
            const int tr = ti < 4 ? 4 * q4 + ti : 16 + 4 * q4 + (ti - 4);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const unsigned a = vcb + tr * CROW + 16 * vslot<D>(tr, nb) + 8 * (s16 & 1);
                asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(vt[nb]) : "v"(a) : "memory");
            }
            if constexpr (NB == 8) {
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(vpw[0]), "+v"(vpw[1]), "+v"(vpw[2]), "+v"(vpw[3]), "+v"(vt[0]), "+v"(vt[1]),
                               "+v"(vt[2]), "+v"(vt[3]), "+v"(vt[4]), "+v"(vt[5]), "+v"(vt[6]), "+v"(vt[7])
                             :
                             : "memory");
            } else {
                static_assert(NB == 4, "head_dim 64 or 128");
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(vpw[0]), "+v"(vpw[1]), "+v"(vpw[2]), "+v"(vpw[3]), "+v"(vt[0]), "+v"(vt[1]),
                               "+v"(vt[2]), "+v"(vt[3])
                             :
                             : "memory");
            }
        }
        // the V stage is free once those reads are done: the next tile's V
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        load_tensor(std::false_type{}, base + kStep, tb_next);
        if constexpr (GP) {
            if (phase == 0) {
                load_pair_group(std::true_type{}, base + kGrp * kStep, gsel ^ 1);
                load_pair_group(std::false_type{}, base + kGrp * kStep, gsel ^ 1);
            }
        }

        float vstep[NS], vzp[NS];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint4 w = __builtin_bit_cast(uint4, vpw[2 * kb + e / 2]);
                vstep[4 * kb + e] = __builtin_bit_cast(float, e % 2 ? w.z : w.x);
                vzp[4 * kb + e] = __builtin_bit_cast(float, e % 2 ? w.w : w.y);
            }

        // online softmax per head (lazy reference max, as in the bf16 kernel);
        // the PV weights are p * step_v, entered as bf16 hi + lo, and the
        // correction sums (hi + lo) * zp_v, rescaled with O and l
        uint32_t ph[HB][NS / 2], pl[HB][NS / 2];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            float mt = s[hb][0];
#pragma unroll
            for (int e = 1; e < NS; ++e) mt = fmaxf(mt, s[hb][e]);
            mt = max_same_head(mt);
            const bool move = mt > m[hb] + kLazy;
            if (__any(move)) {
                const float m_new = move ? mt : m[hb];
                const float alpha = fast_exp2(m[hb] - m_new);
                m[hb] = m_new;
                l[hb] *= alpha;
                corr[hb] *= alpha;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[hb][nb] *= alpha;
            }
            float pw[NS], ps = 0.0f;
#pragma unroll
            for (int e = 0; e < NS; ++e) {
                const float pr = fast_exp2(s[hb][e] - m[hb]);
                ps += pr;
                pw[e] = pr * vstep[e];
            }
#pragma unroll
            for (int i = 0; i < NS / 2; ++i) {
                ph[hb][i] = pack2_bf16(pw[2 * i], pw[2 * i + 1]);
                pl[hb][i] = pack2_bf16(pw[2 * i] - bf16_lo(ph[hb][i]), pw[2 * i + 1] - bf16_hi(ph[hb][i]));
                if constexpr (ZP) {
                    corr[hb] = fmaf(bf16_lo(ph[hb][i]) + bf16_lo(pl[hb][i]), vzp[2 * i], corr[hb]);
                    corr[hb] = fmaf(bf16_hi(ph[hb][i]) + bf16_hi(pl[hb][i]), vzp[2 * i + 1], corr[hb]);
                }
            }
            l[hb] += ps;
        }

        // O^T += V^T P^T: the transposed codes converted to bf16 (exact), one
        // 16x16x32 product per column block and weight term
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint4 va = codes8_to_bf16<FMT>(__builtin_bit_cast(uint2, vt[nb]));
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                o[hb][nb] = mfma16(va, make_uint4(ph[hb][0], ph[hb][1], ph[hb][2], ph[hb][3]), o[hb][nb]);
                o[hb][nb] = mfma16(va, make_uint4(pl[hb][0], pl[hb][1], pl[hb][2], pl[hb][3]), o[hb][nb]);
            }
        }
    };

    // Tiles past the split are loaded anyway (zero range: no memory access), so
    // every path has the same loads in flight and the waits stay exact.
    if (base < t_end) {
        for (int tile = 0;; ++tile) {
            compute_tile(base, tile % kGrp, (tile / kGrp) & 1);
            base += kStep;
            if (base >= t_end) break;
        }
    }

    // ---- apply the zero-point correction and merge the waves (LDS reused
    // once every load of this workgroup has landed)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        l[hb] = sum_same_head(l[hb]);
        if constexpr (ZP) {
            const float c = sum_same_head(corr[hb]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[hb][nb] -= c;
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    if constexpr (FUSED) {
        // Results of the append, stored once every load of this workgroup has
        // completed: the rotated query (split 0) and the new token's codes and
        // pairs (the split that holds it; it patched them into its tile).
        const bool qout = split == 0 && wave == 0 && p.q_rot_out != nullptr;
        const __amdgpu_buffer_rsrc_t qors =
            make_uniform_rsrc(qout ? static_cast<uint16_t*>(p.q_rot_out) + qgrp : p.q_rot_out, qout ? G * D * 2 : 0);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, qb[hb][kk]), qors,
                                                       ((16 * hb + r16) * D + 32 * kk + 8 * q4) * 2, 0, 0);
        const bool st = slot_ok && wave == 0 && r16 == 0;
        const __amdgpu_buffer_rsrc_t kcs = make_uniform_rsrc(static_cast<uint8_t*>(const_cast<void*>(p.k)) + slot_row * D,
                                                             slot_ok ? D : 0);
        const __amdgpu_buffer_rsrc_t vcs = make_uniform_rsrc(static_cast<uint8_t*>(const_cast<void*>(p.v)) + slot_row * D,
                                                             slot_ok ? D : 0);
        if (st) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, kcode[kk]), kcs, 32 * kk + 8 * q4, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, vcode[kk]), vcs, 32 * kk + 8 * q4, 0, 0);
            }
        }
        if (slot_ok && tid == 0) {
            *reinterpret_cast<float2*>(k_sz + slot_row * 2) = kpair;
            *reinterpret_cast<float2*>(v_sz + slot_row * 2) = vpair;
        }
    }

    // O rows of the group's heads through LDS, RB rows per pass (chunks of row
    // r XOR-swizzled by r mod 16: the 16 lanes of one 128-bit store, one
    // column chunk of 16 rows, fill one 256-byte sweep of the banks); one
    // thread per 16-byte column chunk of a row
    constexpr int RB = (2 * CSTAGE / (4 * D)) < 16 ? (2 * CSTAGE / (4 * D)) : 16;
    constexpr int NCH = D / 4;
    static_assert(RB >= 4 && NW * RB * D * 4 <= 2 * NW * CSTAGE, "merge area");
    static_assert(NCH >= 16, "16 swizzle slots per row");
    auto chunk_at = [](int row, int ch) { return ch ^ (row & 15); };
    // (the in-kernel merge's partials: offsets below 2^31, as planned)
    const __amdgpu_buffer_rsrc_t part_rs = make_uniform_rsrc(p.ws_part, 0x7FFFFFFF);
    const __amdgpu_buffer_rsrc_t ml_rs = make_uniform_rsrc(p.ws_ml, 0x7FFFFFFF);
    float* sm_o = reinterpret_cast<float*>(code_lds);             // [NW][RB][D]
    float* sm_m = reinterpret_cast<float*>(ksz_lds);              // [NW][16]
    float* sm_l = sm_m + NW * 16;                                   // [NW][16]
    const int NT = NW * 64;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        if (q4 == 0) {
            sm_m[wave * 16 + r16] = m[hb];
            sm_l[wave * 16 + r16] = l[hb];
        }
        const int heads = min(16, G - 16 * hb);
        for (int r0 = 0; r0 < heads; r0 += RB) {
            const int row = r16 - r0;
            if (row >= 0 && row < RB && r16 < heads) {
                float* dst = sm_o + (wave * RB + row) * D;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    *reinterpret_cast<float4*>(dst + 4 * chunk_at(row, 4 * nb + q4)) =
                        make_float4(o[hb][nb][0], o[hb][nb][1], o[hb][nb][2], o[hb][nb][3]);
            }
            __syncthreads();
            const int rows = min(RB, heads - r0);
            for (int idx = tid; idx < rows * NCH; idx += NT) {
                const int gr = idx / NCH;
                const int ch = idx % NCH;
                const int gh = r0 + gr;
                const int at = 4 * chunk_at(gr, ch);
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * 16 + gh]);
                float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                float Ls = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float mw = sm_m[w * 16 + gh];
                    const float f = (mw == -kNoMax) ? 0.0f : fast_exp2(mw - M);
                    const float4 ow = *reinterpret_cast<const float4*>(sm_o + (w * RB + gr) * D + at);
                    A.x = fmaf(ow.x, f, A.x);
                    A.y = fmaf(ow.y, f, A.y);
                    A.z = fmaf(ow.z, f, A.z);
                    A.w = fmaf(ow.w, f, A.w);
                    Ls = fmaf(sm_l[w * 16 + gh], f, Ls);
                }
                const size_t bh = static_cast<size_t>(b) * p.H_q + j * G + 16 * hb + gh;
                const int c = 4 * ch;
                if (nsp == 1) {
                    uint2 packed;
                    packed.x = static_cast<uint32_t>(f32_to_bf16_rne(Ls > 0.0f ? A.x / Ls : 0.0f)) |
                               (static_cast<uint32_t>(f32_to_bf16_rne(Ls > 0.0f ? A.y / Ls : 0.0f)) << 16);
                    packed.y = static_cast<uint32_t>(f32_to_bf16_rne(Ls > 0.0f ? A.z / Ls : 0.0f)) |
                               (static_cast<uint32_t>(f32_to_bf16_rne(Ls > 0.0f ? A.w / Ls : 0.0f)) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + bh * D + c) = packed;
                } else if (p.merge_cnt != nullptr) {
                    // device-scope stores (written through to memory that
                    // every XCD sees), for the merge below
                    const size_t pr = BAL ? sg.row + 16 * hb + gh : bh * p.n_splits + split;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, A), part_rs,
                                                           static_cast<int>((pr * D + c) * 4), 0, kDevScope);
                    if (ch == 0)
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, make_float2(M, Ls)),
                                                              ml_rs, static_cast<int>(pr * 8), 0, kDevScope);
                } else {
                    *reinterpret_cast<float4*>(p.ws_part + (bh * p.n_splits + split) * D + c) = A;
                    if (ch == 0) p.ws_ml[bh * p.n_splits + split] = make_float2(M, Ls);
                }
            }
            __syncthreads();
        }
    }

    // ---- merge of the unit's splits by the last of them to finish (as in
    // the bf16 kernel: device-scope partial rows, a wrapping arrival count,
    // no workgroup waiting for another)
    if (nsp > 1 && p.merge_cnt != nullptr) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        if (tid == 0)
            s_last = __builtin_amdgcn_atomic_inc32(p.merge_cnt + unit, static_cast<unsigned>(nsp - 1),
                                                   __ATOMIC_RELAXED, "agent") == static_cast<unsigned>(nsp - 1);
        __syncthreads();
        if (!s_last) continue;
        const size_t row0 = static_cast<size_t>(b) * p.H_q + static_cast<size_t>(j) * G;
        merge_split_rows<D>(p, part_rs, ml_rs, G, nsp, [&](int gr) -> size_t { return row0 + gr; },
                            [&](int gr, int s) -> size_t {
                                if constexpr (BAL) return bal_part_row(p, sg, gr, s);
                                else return (row0 + gr) * p.n_splits + s;
                            });
    }
    }   // segments
}

template <int D, int HB, bool FUSED, int FMT>
hipError_t launch_dhff(bool paged, const DecodeParams& p, float* k_sz, float* v_sz, hipStream_t stream,
                       const KernelTiming& tm) {
    const dim3 grid(p.n_wg_pad), block(kNWq * 64);
    if (p.bal) {
        // balanced schedule: planned for paged pools of at most kBalMaxB sequences
        if (!paged || p.B > kBalMaxB) return hipErrorInvalidValue;
        return launch_timed(decode_u8_kernel<D, HB, 3, FUSED, true, FMT>, grid, block, stream, tm, p, p.block_table,
                            k_sz, v_sz);
    }
    if (paged)
        return launch_timed(decode_u8_kernel<D, HB, 3, FUSED, false, FMT>, grid, block, stream, tm, p, p.block_table,
                            k_sz, v_sz);
    return launch_timed(decode_u8_kernel<D, HB, 0, FUSED, false, FMT>, grid, block, stream, tm, p, p.block_table,
                        k_sz, v_sz);
}

template <int D, int HB, bool FUSED>
hipError_t launch_dhf(bool paged, int qfmt, const DecodeParams& p, float* k_sz, float* v_sz, hipStream_t stream,
                      const KernelTiming& tm) {
    switch (qfmt) {
        case kQ8Affine: return launch_dhff<D, HB, FUSED, kQ8Affine>(paged, p, k_sz, v_sz, stream, tm);
        case kQ8E4M3: return launch_dhff<D, HB, FUSED, kQ8E4M3>(paged, p, k_sz, v_sz, stream, tm);
        case kQ8E5M2: return launch_dhff<D, HB, FUSED, kQ8E5M2>(paged, p, k_sz, v_sz, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int HB>
hipError_t launch_dh(bool paged, bool fused, int qfmt, const DecodeParams& p, float* k_sz, float* v_sz,
                     hipStream_t stream, const KernelTiming& tm) {
    return fused ? launch_dhf<D, HB, true>(paged, qfmt, p, k_sz, v_sz, stream, tm)
                 : launch_dhf<D, HB, false>(paged, qfmt, p, k_sz, v_sz, stream, tm);
}

}  // namespace

bool decode_u8_supported(int d, int G) { return (d == 64 || d == 128) && G >= 1 && G <= 32; }

int decode_u8_step_tokens() { return kNWq * kTTq; }

int decode_u8_wgs_per_cu(int d, int G) {
    // LDS per workgroup: code tiles 2 * 4 * 32 * d, pair rows 2 KiB (+ 4 KiB
    // of table when paged): 34-40 KiB at d = 128; registers (about 180 per
    // lane with one 16-head block, 280 with two) allow two waves per SIMD, or
    // one, so two workgroups per CU, or one.
    (void)d;
    return G > 16 ? 1 : 2;
}

hipError_t launch_decode_u8(int d, int G, bool paged, bool fused, int qfmt, const DecodeParams& p, float* k_sz,
                            float* v_sz, hipStream_t stream, const KernelTiming& tm) {
    const bool two = G > 16;
    switch (d) {
        case 64:
            return two ? launch_dh<64, 2>(paged, fused, qfmt, p, k_sz, v_sz, stream, tm)
                       : launch_dh<64, 1>(paged, fused, qfmt, p, k_sz, v_sz, stream, tm);
        case 128:
            return two ? launch_dh<128, 2>(paged, fused, qfmt, p, k_sz, v_sz, stream, tm)
                       : launch_dh<128, 1>(paged, fused, qfmt, p, k_sz, v_sz, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
