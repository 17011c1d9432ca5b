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
// * The probabilities enter the second product as three bf16 operands
//   (hi = bf16(p), mid = bf16(p - hi), lo = bf16(p - hi - mid)), three MFMAs,
//   so p carries about 24 significant bits, as a float32 weight would (the
//   32-row multi-token kernel: hi and mid only, for want of registers).  One
//   bf16 operand alone leaves errors of a few 1e-4 in the output; two (about
//   16 bits, relative error up to ~4e-6 per weight) still moved outputs of
//   short sequences with |O| >= 0.5 across a bf16 rounding boundary now and
//   then (one bf16 step there is 3.9e-3).

#include <type_traits>

#include "kvc_internal.h"
#include "kvc_device.h"
#include "kvc_mfma_common.h"

namespace kvc {

namespace {

using namespace mfma;


// MODE 0: contiguous cache.  MODE 1: paged, any block size (each row's block
// looked up per lane).  MODE 2: paged with block_size % 16 == 0 and splits
// starting on 32-token boundaries, so every 16-row group of a tile lies in one
// block: one wave-uniform table lookup per group.  MODE 3: paged, d <= 128,
// block_size % 16 == 0, splits starting on 16-token boundaries and spanning at
// most kTblMax blocks: the split's slice of the block table is staged in LDS
// once, and K and V tiles are staged like those of a contiguous cache.
// (The paged kernel with staged tiles and one head block is planned at three
// workgroups per CU: its registers are held to three waves per SIMD.)
template <int D, int HB, int NW, int MODE, bool FUSED, bool MQ, bool BAL>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu((MODE == 3 && HB == 1) ? 3 : ((HB == 2 && MODE == 0 && D <= 128) ? 2 : 1), 8)))
decode_mfma_kernel(const DecodeParams p, const int32_t* __restrict__ block_table) {
    // (the block table as its own restrict argument: nothing this kernel stores
    // can alias it, so its wave-uniform reads may use scalar loads)
    constexpr bool PAGED = MODE != 0;
    constexpr int KK = D / 32;            // 32-wide d slices per 16-token block
    constexpr int NB = D / 16;            // 16-column blocks of V
    // K tiles are staged in LDS up to d = 128 (contiguous caches, and paged
    // ones in MODE 3): a direct load moves whole 256-byte rows, while loading
    // K straight into the MFMA operand moves 64-byte pieces of 16 rows per
    // instruction, which streamed about 4 % slower.  (MODE 2 keeps K in
    // registers: there, staging K doubled its per-group scalar table reads,
    // which the halved occupancy could not hide - measured twice as slow.)
    constexpr bool KLDS = D <= 128 && (MODE == 0 || MODE == 3);
    // Stages per wave of staged K and V tiles.  The 32 query rows of several
    // new tokens do twice the matrix and softmax work per tile of a 16-row
    // head block, which a single stage's refill latency then adds to: over a
    // contiguous cache they get two stages (tile i + 2 loads while tile i is
    // computed; spec_gqa 100.9 -> 91.3 us).  (A single-token group of 32
    // heads, whose fused prologue leaves fewer registers, measured slower so.)
    constexpr int NSTG = (KLDS && MQ && HB == 2 && MODE == 0) ? 2 : 1;
    // Tokens per wave tile: 16 where K is staged, else 32.  Half-height tiles
    // keep 8 KiB per wave (32 KiB per CU) in flight while a wave waits, the
    // amount a plain streaming read needed for its best rate on this part;
    // 32-row tiles doubled that and were slower.
    constexpr int TT = KLDS ? 16 : 32;
    constexpr int KB = TT / 16;           // 16-row K blocks per tile
    constexpr int ROWB = 2 * D;           // LDS bytes per staged V row
    constexpr int STAGE = TT * ROWB;      // LDS bytes of one V tile
    // With K staged, each wave has one K and one V stage, each refilled as
    // soon as the tile's computation is done with it (K after its operand
    // reads, V after the PV product): at most one tile's K and V in flight,
    // which streamed about 2 % faster than two full stages.  With K in
    // registers, V is double-buffered per wave in two separate arrays (so
    // the compiler can tell the tile being read from the one being filled)
    // and K uses two operand arrays.
    __shared__ __attribute__((aligned(16))) char vbuf0[NW * STAGE];
    __shared__ __attribute__((aligned(16))) char vbuf1[(KLDS && NSTG == 1) ? 16 : NW * STAGE];
    __shared__ __attribute__((aligned(16))) char kbuf[KLDS ? NW * STAGE : 16];
    __shared__ __attribute__((aligned(16))) char kbuf1[NSTG == 2 ? NW * STAGE : 16];
    __shared__ int tbl_lds[MODE == 3 ? kTblMax : 1];
    __shared__ float sm_ml[2 * NW * 16];   // the waves' (m, l) per head row, for their merge

    __shared__ int s_last;                 // the in-kernel merge: this workgroup arrived last
    __shared__ std::conditional_t<BAL, BalLds, char> bal;   // the balanced schedule's lengths and prefix

    const int wid = blockIdx.x < static_cast<unsigned>(p.n_wg) ? static_cast<int>(blockIdx.x) : -1;
    if (wid < 0) return;
    const int G = p.G;
    static_assert(!(MQ && FUSED), "several new tokens: the append runs first");
    static_assert(!(BAL && MQ), "the balanced schedule serves single-token steps");
    constexpr int kStep = NW * TT;        // tokens per loop step of the workgroup
    constexpr bool CMP = MODE == 0 && !MQ && !BAL;   // compacted numbering available (p.compact)

    const int tid0 = threadIdx.x;

    // Balanced schedule (paged pools with ragged lengths; the helpers in
    // kvc_mfma_common.h): every workgroup reads all lengths, then runs its
    // split body once per segment of its equal share of all units' steps.
    if constexpr (BAL) {
        if (!bal_setup<NW * 64, kStep, FUSED>(p, wid, bal)) return;
    }

    // MODE 3 without a window (split schedule): the split's first block is
    // known before its sequence's length (the split starts at split *
    // split_tokens), so the table entries it may span are requested together
    // with the length, and the first tile waits for one round trip less.
    // (Entries past the row are clamped into it; those past the split are not
    // used.)
    constexpr int kTblPer = kTblMax / (NW * 64);
    int tv[kTblPer];
    const bool tbl_early = MODE == 3 && p.window == 0 && !BAL;

    // (one pass under the split schedule: a trip count the compiler can see
    // keeps its register allocation that of straight-line code)
    for (int it = 0; BAL || it < 1; ++it) {
    // ---- one split (balanced schedule: one segment) of one unit
    int unit, split, nsp, t_begin, t_end, t_lo, L, pos;
    BalSeg sg{};                          // balanced schedule: this segment
    if constexpr (BAL) {
        if (!bal_segment<kStep, FUSED>(p, wid, it, bal, sg)) break;
        unit = sg.unit;
        nsp = sg.nsp;
        split = sg.split;
        L = sg.L;
        pos = sg.pos;
        t_begin = sg.t_begin;
        t_end = sg.t_end;
        t_lo = 0;
        // (the previous segment's output stores, before this one's loads)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else if (CMP && p.compact) {
        // Compacted schedule (contiguous cache, plans of several rounds; the
        // helper in kvc_mfma_common.h): the split length comes from the
        // lengths themselves, and the splits that exist take the first
        // workgroup indices.
        CmpSeg c;
        if (!cmp_locate<FUSED>(p, wid, c)) return;
        unit = c.unit;
        split = c.split;
        nsp = c.nsp;
        L = c.L;
        pos = c.pos;
        if (split == 0 && tid0 == 0 && p.ws_nsp != nullptr) p.ws_nsp[unit] = nsp;   // for the merge kernel
        const TokenRange tr = token_range(p, L);
        t_begin = tr.org + split * c.T;
        const int e = tr.org + (split + 1) * c.T;
        t_end = (split == nsp - 1 || e > tr.hi) ? tr.hi : e;
        t_lo = tr.lo;
    } else {
        // Workgroups in launch order: the splits of one (sequence, KV head)
        // are neighbours, and the hardware deals consecutive workgroups to the
        // XCDs in turn.  (Grouping each unit's splits on one XCD gains nothing
        // for a stream without reuse, and with ragged lengths it left some
        // XCDs with far more work than others: the paged workload ran 2.4 %
        // slower.)
        split = wid % p.n_splits;
        unit = wid / p.n_splits;          // b * H_kv + j (MQ: (b * H_kv + j) * n_chunks + chunk)
        if constexpr (MODE == 3) {
            if (tbl_early) {
                const int b0 = (MQ ? unit / p.n_chunks : unit) / p.H_kv;
                const int fb0 = (split * p.split_tokens) / p.block_size;
                const int span = min(p.split_tokens / p.block_size + 1, p.max_blocks_per_seq - fb0);
                const int32_t* trow = block_table + static_cast<size_t>(b0) * p.max_blocks_per_seq;
                const int first = min(fb0, p.max_blocks_per_seq - 1);
#pragma unroll
                for (int k = 0; k < kTblPer; ++k) {
                    const int i = tid0 + k * NW * 64;
                    tv[k] = trow[i < span ? fb0 + i : first];
                }
            }
        }
        const int b0 = (MQ ? unit / p.n_chunks : unit) / p.H_kv;
        // fused step: slot of the new token (read once; it also gives L)
        pos = FUSED ? p.positions[b0] : 0;
        L = FUSED ? len_from_position(p, pos) : attended_len(p, b0);
        // attended tokens [t_lo, hi) (a sliding window starts past 0); the
        // paged modes start their splits at t_lo rounded down to 16 and read
        // the rows before t_lo as zeros (out-of-range offsets) or as row
        // t_lo, masked
        const TokenRange tr = token_range(p, L);
        nsp = split_count(p, tr);
        if (split >= nsp) return;
        t_begin = tr.org + split * p.split_tokens;
        t_end = split_end(p, tr, split, nsp);
        t_lo = tr.lo;
    }
    // The lane index, opaque to the compiler inside each segment of the
    // balanced schedule: the per-lane offsets derived from it are then
    // computed per segment rather than hoisted above the segment loop, where
    // they would stay live through every epilogue (about 50 registers more).
    int tid = tid0;
    if constexpr (BAL) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = MQ ? unit % p.n_chunks : 0;
    const int bj = MQ ? unit / p.n_chunks : unit;
    const int b = bj / p.H_kv;
    const int j = bj % p.H_kv;

    const int r16 = lane & 15;            // row/column index inside the operand
    const int q4 = lane >> 4;             // 16-lane group: reduction slots 8*q4 .. +7

    float m[HB], l[HB];
    f32x4_t o[HB][NB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        // finite start: a tile whose rows are all masked (possible with the
        // interleaved rows) then gives weights 2^(-inf - m) = 0, not NaN
        m[hb] = -kNoMax;
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
    // K rows: chunk c at slot c ^ (r % LPR), so the 16 lanes reading one
    // chunk of 16 consecutive rows for the MFMA operand hit distinct banks
    auto swzk = [](int r) { return r & (LPR - 1); };

    // Token of row r of this wave's tile at step base.  With K staged in LDS
    // the waves interleave: in every 16-token group, wave w takes 4 tokens
    // (row r -> base + 16 * (r / 4) + 4 * w + r % 4), so one load instruction
    // of each of the 4 waves covers 16 consecutive rows and the workgroup
    // reads its K and V as two sequential streams (a wave streaming its own
    // 32-row block was measurably slower).  Otherwise each wave takes 32
    // consecutive tokens from its own base.
    // (Paged tiles are not interleaved: each wave's 16 rows then lie in one
    // block, found with one table lookup.)
    constexpr bool ILV = KLDS && MODE == 0;
    static_assert(!ILV || NW == 4, "interleaved rows assume four waves");
    auto tok = [&](int base, int r) __attribute__((always_inline)) {
        return ILV ? base + 16 * (r >> 2) + 4 * wave + (r & 3) : base + r;
    };

    // Contiguous caches are read through buffer resources whose range ends at
    // row t_end of this (sequence, KV head): rows past the split read as zeros
    // without touching memory, so no clamping is needed.  Paged caches clamp
    // the row to t_end - 1 (always a valid, finite row of this sequence).
    // In the fused step the new token's row is patched into its tile from
    // registers (below), so the range of the split holding it stops before
    // that row: it is never read, and a last step holding only it reads
    // nothing from memory.
    const bool patch_new = FUSED && MODE == 0 && split == nsp - 1 && pos >= 0 && pos < p.capacity &&
                           pos < p.rope_rows && pos < t_end;
    const size_t rows_bytes = static_cast<size_t>(patch_new ? pos : t_end) * D * 2;
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

    // MODE 3: buffer resource of the wave's 16-row tile at row0 (wave-uniform,
    // a multiple of 16, so the rows lie in one block), its block id read from
    // the staged table slice; its range ends at the last row < t_end, so rows
    // past the split read as zeros without a memory access.
    const int fb = PAGED ? t_begin / p.block_size : 0;   // first block index of the split
    // (the block id of the tile at row0, read from the staged slice; a tile's
    // K and V rows share it, so the tile computation reads it once, early,
    // for the tile it refills)
    auto tile_block = [&](int row0_) -> int {
        const int row0 = __builtin_amdgcn_readfirstlane(row0_);
        int ti = row0 / p.block_size - fb;
        ti = ti < 0 ? 0 : (ti >= kTblMax ? kTblMax - 1 : ti);
        return tbl_lds[ti];
    };
    auto tile_rsrc = [&](const uint16_t* pool, int row0_, int blk_) -> __amdgpu_buffer_rsrc_t {
        const int row0 = __builtin_amdgcn_readfirstlane(row0_);
        int nvalid = __builtin_amdgcn_readfirstlane(t_end) - row0;
        nvalid = nvalid < 0 ? 0 : (nvalid > 16 ? 16 : nvalid);
        const int lb = row0 / p.block_size;
        const int blk = __builtin_amdgcn_readfirstlane(nvalid > 0 ? blk_ : 0);
        const int in_blk = row0 - lb * p.block_size;
        const uint16_t* g0 = pool + ((static_cast<size_t>(blk) * p.H_kv + j) * p.block_size + in_blk) * D;
        return make_uniform_rsrc(g0, nvalid * D * 2);
    };

    // K rows of a tile, straight into A operands (registers)
    auto load_k = [&](int base, uint4 (&ka)[KB][KK]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int t = tok(base, 16 * kb + r16);
            if constexpr (MODE == 2) {
                const __amdgpu_buffer_rsrc_t rs = group_rsrc(kbase, base + 16 * kb);
                const int off = ((t < t_lo ? 16 : r16) * D + 8 * q4) * 2;   // rows before the window: past the range
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * kk, 0, kNT));
            } else if constexpr (PAGED) {
                const size_t off = row_off(t < t_lo ? t_lo : (t < t_end ? t : t_end - 1)) + 8 * q4;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(kbase + off + 32 * kk)));
            } else {
                const int off = (t * D + 8 * q4) * 2;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64 * kk, 0, kNT));
            }
        }
    };
    // Rows of a tile (V, and K when KLDS), HBM -> LDS without passing through
    // registers: lane l of load i fills LDS bytes [16 l, 16 l + 16) of that
    // load's 1 KiB, i.e. row VROWS*i + l / LPR, slot l % LPR, so it fetches
    // chunk (slot ^ swizzle(row)).
    auto load_rows = [&](auto is_k, int base, char* buf, int blk_) __attribute__((always_inline)) {
        constexpr bool ISK = decltype(is_k)::value;
        const uint16_t* pool = ISK ? kbase : vbase;
        char* wbuf = buf + wave * STAGE;
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int r = VROWS * i + lane / LPR;
            const int u = (lane % LPR) ^ (ISK ? swzk(r) : swz(r));
            const int t = tok(base, r);
            lds_void_t* dst = (lds_void_t*)(wbuf + 1024 * i);
            // (rows before the window's first token get an offset past the
            // 16-row range, so they read as zeros without a memory access)
            if constexpr (MODE == 3) {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(pool, base, blk_);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ((t < t_lo ? 16 : r) * D + 8 * u) * 2, 0, 0,
                                                         kNT);
            } else if constexpr (MODE == 2) {
                const int row0 = (VROWS * i / 16) * 16;           // this load's 16-row group
                const __amdgpu_buffer_rsrc_t rs = group_rsrc(pool, base + row0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, ((t < t_lo ? 16 : r - row0) * D + 8 * u) * 2, 0,
                                                         0, kNT);
            } else if constexpr (PAGED) {
                const uint16_t* src = pool + row_off(t < t_lo ? t_lo : (t < t_end ? t : t_end - 1)) + 8 * u;
                __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kNT);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ISK ? krs : vrs, dst, 16, (t * D + 8 * u) * 2, 0, 0, kNT);
            }
        }
    };
    // one tile: K (LDS or registers), then V
    auto load_tile = [&](int base, uint4 (&ka)[KB][KK], char* kb, char* vb) __attribute__((always_inline)) {
        const int blk = MODE == 3 ? tile_block(base) : 0;
        if constexpr (KLDS) load_rows(std::true_type{}, base, kb, blk);
        else load_k(base, ka);
        load_rows(std::false_type{}, base, vb, blk);
    };
    // K operand of a tile staged in LDS: lane (r16, q4) takes 16-byte chunk
    // 4*kk + q4 of rows r16 and 16 + r16 (the layout load_k produces)
    auto read_k = [&](const char* kb, uint4 (&ka)[KB][KK]) __attribute__((always_inline)) {
        const char* wk = kb + wave * STAGE;
#pragma unroll
        for (int h = 0; h < KB; ++h) {
            const int r = 16 * h + r16;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                ka[h][kk] = *reinterpret_cast<const uint4*>(wk + r * ROWB + 16 * ((4 * kk + q4) ^ swzk(r)));
        }
    };

    // Prologue.  The small loads go out first (the query and, in the fused
    // step, the new token and its rotation table row), then the first tile:
    // loads complete in order, so the rotation waits for the small loads
    // only and runs while the tile is in flight.
    int base = t_begin + (ILV ? 0 : wave * TT);   // step base: the workgroup's, or this wave's
    uint4 ka0[KB][KK], ka1[KB][KK];

    // MODE 3 with a window: the table entries of the blocks this split spans
    // (read first: the first tile's addresses depend on them).  Indices past
    // the split are clamped to its first entry, so every read stays in this
    // sequence's row.
    const int nblk = PAGED ? (t_end - 1) / p.block_size - fb + 1 : 0;
    if constexpr (MODE == 3) {
        if (!tbl_early) {
#pragma unroll
            for (int k = 0; k < kTblPer; ++k) {
                const int i = tid + k * NW * 64;
                tv[k] = table[fb + (i < nblk ? i : 0)];
            }
        }
    }

    // B operand Q^T: lane holds head 16*hb + r16, d = 32*kk + 8*q4 .. +7.  The
    // group's G query rows are read through a buffer resource covering exactly
    // them, so lanes of heads >= G read zeros.
    const size_t qgrp = (static_cast<size_t>(b) * p.H_q + static_cast<size_t>(j) * G) * D;
    const __amdgpu_buffer_rsrc_t qrs =
        MQ ? make_uniform_rsrc(static_cast<const uint16_t*>(p.q) + static_cast<size_t>(b) * p.qlen * p.H_q * D,
                               p.qlen * p.H_q * D * 2)
           : make_uniform_rsrc(static_cast<const uint16_t*>(FUSED ? p.q_raw : p.q) + qgrp, G * D * 2);
    // MQ: this lane's query row of each head block is row rho of the group's
    // G * qlen rows (new token i = rho / G, head g = rho % G) at
    // q[b, i, j * G + g]; rows past the last read zeros (offset past the range)
    int qoff[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        if constexpr (MQ) {
            const int rho = chunk * 16 * HB + 16 * hb + r16;
            const int qi = rho / G;
            qoff[hb] = rho < G * p.qlen ? (qi * p.H_q + j * G + (rho - qi * G)) * D : p.qlen * p.H_q * D;
        } else {
            qoff[hb] = (16 * hb + r16) * D;
        }
    }
    uint4 qb[HB][KK];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qb[hb][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                qrs, (qoff[hb] + 32 * kk + 8 * q4) * 2, 0, 0));
    // MQ: tokens this lane's query rows attend, [row_lo, row_hi) within the
    // split: causal among the new tokens (token i sees up to L - qlen + i),
    // and its own window start
    int row_lo[HB], row_hi[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        if constexpr (MQ) {
            const int rho = chunk * 16 * HB + 16 * hb + r16;
            const int hi = L - p.qlen + rho / G + 1;
            const int lo = p.window > 0 ? max(0, hi - p.window) : 0;
            row_hi[hb] = min(t_end, hi);
            row_lo[hb] = max(t_lo, lo);
        } else {
            row_hi[hb] = t_end;
            row_lo[hb] = t_lo;
        }
    }

    // Fused step.  The new token sits at slot pos of sequence b; the last
    // split of (b, j) stores it (rotated key, raw value) and, since its own
    // tile loads may run before or after that store, patches the token into
    // the tile it loaded instead of reading it back: the key row in the K
    // operand, the value row in the staged V tile.  Every wave issues the
    // same memory instructions whatever its role; a role it does not have
    // gets a buffer range of zero bytes (loads read zeros, stores are
    // dropped), so the waits of the tile pipeline stay exact.
    const bool pos_ok = FUSED && pos >= 0 && pos < p.capacity && pos < p.rope_rows;
    const bool own = pos_ok && split == nsp - 1;
    const bool half = FUSED && p.rope_style == KVC_ROPE_HALF;
    uint4 kn[KK];                         // rotated new key, A-operand layout
    uint4 vn = make_uint4(0, 0, 0, 0);    // raw new value, 16-byte chunk lane % LPR
    float4 cw[KK], sw[KK];                // cos/sin of the pairs this lane's chunks hold
    if constexpr (FUSED) {
        const size_t kv_in = (static_cast<size_t>(b) * p.H_kv + j) * D;
        const __amdgpu_buffer_rsrc_t knrs =
            make_uniform_rsrc(static_cast<const uint16_t*>(p.k_new) + kv_in, own ? D * 2 : 0);
        const __amdgpu_buffer_rsrc_t vnrs =
            make_uniform_rsrc(static_cast<const uint16_t*>(p.v_new) + kv_in, own ? D * 2 : 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            kn[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                knrs, (32 * kk + 8 * q4) * 2, 0, 0));
        vn = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vnrs, (lane % LPR) * 16, 0, 0));

        // Adjacent pairs: chunk kk holds pairs 16*kk + 4*q4 .. +3.  Split
        // halves: chunks m and m + KK/2 pair up element by element, pairs
        // 32*m + 8*q4 .. +7, kept as cw[2m], cw[2m + 1].  (Row 0 stands in
        // when the position is invalid: the query is then left as it is and
        // nothing is stored.)
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

    // (unconditional, like every tile load: a wave with nothing to do reads
    // zeros or the clamped last row.  Behind a branch, the compiler's own
    // waits for the small loads would assume the path without these loads
    // and wait for the tile as well.)
    if constexpr (MODE == 3) {
        // (ids out of range are clamped into the pool, so no access leaves
        // it; in-range ids are the caller's contract)
#pragma unroll
        for (int k = 0; k < kTblPer; ++k) {
            const int i = tid + k * NW * 64;
            const int blk = tv[k] < 0 ? 0 : (tv[k] >= p.num_blocks ? p.num_blocks - 1 : tv[k]);
            if (i < nblk) tbl_lds[i] = blk;
        }
        __syncthreads();
    }
    load_tile(base, ka0, kbuf, vbuf0);
    if constexpr (NSTG == 2) load_tile(base + kStep, ka0, kbuf1, vbuf1);

    int patch_row = -1;                   // token index of the patched row, or -1
    size_t slot = 0;                      // element offset of the new token's row
    bool slot_ok = false;                 // this split stores the new token
    if constexpr (FUSED) {
        auto fget = [](const float4& v, int i) __attribute__((always_inline)) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; };
        // rotate one vector held as KK chunks, exactly as the append kernel
        // does (float32, one rounding per operation, then bf16 RNE)
        auto rotate = [&](uint4 (&x)[KK]) __attribute__((always_inline)) {
            if (half) {
#pragma unroll
                for (int m = 0; m < KK / 2; ++m) {
                    uint32_t* xa = reinterpret_cast<uint32_t*>(&x[m]);
                    uint32_t* ya = reinterpret_cast<uint32_t*>(&x[m + KK / 2]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int e0 = 2 * w, e1 = 2 * w + 1;     // elements of this dword
                        float a0, a1, b0, b1;
                        rope_pair(bf16_lo(xa[w]), bf16_lo(ya[w]), fget(cw[2 * m + e0 / 4], e0 % 4),
                                  fget(sw[2 * m + e0 / 4], e0 % 4), a0, b0);
                        rope_pair(bf16_hi(xa[w]), bf16_hi(ya[w]), fget(cw[2 * m + e1 / 4], e1 % 4),
                                  fget(sw[2 * m + e1 / 4], e1 % 4), a1, b1);
                        xa[w] = pack_bf16x2(a0, a1);
                        ya[w] = pack_bf16x2(b0, b1);
                    }
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    uint32_t* xa = reinterpret_cast<uint32_t*>(&x[kk]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        float r0, r1;
                        rope_pair(bf16_lo(xa[w]), bf16_hi(xa[w]), fget(cw[kk], w), fget(sw[kk], w), r0, r1);
                        xa[w] = pack_bf16x2(r0, r1);
                    }
                }
            }
        };
        if (pos_ok) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) rotate(qb[hb]);
        }
        rotate(kn);

        // the new token's slot (a clamped table entry would be another
        // sequence's block: then nothing is stored)
        if constexpr (PAGED) {
            if (own) {
                const int blk = table[pos / p.block_size];
                slot_ok = blk >= 0 && blk < p.num_blocks;
                slot = ((static_cast<size_t>(slot_ok ? blk : 0) * p.H_kv + j) * p.block_size + pos % p.block_size) * D;
            }
        } else {
            slot_ok = own;
            slot = seq_off + static_cast<size_t>(own ? pos : 0) * D;
        }

        // the token is attended over (pos < t_end) only when max_seq_len
        // covers it; only the wave whose tile holds it patches
        patch_row = __builtin_amdgcn_readfirstlane(slot_ok && pos < t_end ? pos : -1);
    }

    // transposed-read source of this lane: row tr_row (+16 for the upper half),
    // columns 16*nb + 4*(s16 % 4) .. +3 = chunk 2*nb + (s16 % 4) / 2, half s16 & 1
    const int s16 = lane & 15;
    const int tr_row = 4 * q4 + s16 / 4;

    // Vector memory operations one tile issues: K rows (into LDS, or into
    // registers at d = 256 and for paged caches), then V rows into LDS (paged
    // caches with other block sizes add table reads, which only make the
    // waits below more conservative).
    constexpr int kTileLoads = (KLDS ? VLOADS : 2 * KK) + VLOADS;
    static_assert(VLOADS + kTileLoads < 64, "vmcnt range");
    // Loads issued after this tile's V rows, before its V wait: the next
    // tile's K rows (staged K; with two stages, also the following tile's V
    // and the one after's K), or the whole next tile.
    constexpr int kAfterV = KLDS ? (2 * NSTG - 1) * VLOADS : kTileLoads;
    static_assert(kAfterV < 64, "vmcnt range");

    // A stage is refilled only once every LDS read of it has completed: a
    // direct load writes LDS when its data returns, outside the order of the
    // wave's own LDS instructions, so a read still queued could see the new
    // tile (a load past the split returns almost at once).  The wait also
    // keeps the compiler from moving the refill in among those reads.
    auto compute_tile = [&](uint4 (&ka)[KB][KK], char* kb, char* buf, int base) __attribute__((always_inline)) {
        char* wbuf = buf + wave * STAGE;
        // block id of the tile NSTG steps ahead (paged, staged table): read
        // first, so the wait before the K refill covers it
        const int blk_next = MODE == 3 ? tile_block(base + NSTG * kStep) : 0;
        if constexpr (KLDS) {
            // this tile's K rows were issued before its V rows and nothing
            // after those (two stages: and the next tile's K and V): at most
            // (2 NSTG - 1) VLOADS outstanding
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((2 * NSTG - 1) * VLOADS));
            read_k(kb, ka);
            // the K stage is free once those reads are done: the K rows of
            // the tile NSTG steps ahead go out now (past the split: zeros,
            // no traffic)
            __builtin_amdgcn_s_waitcnt(kLgkmZero);
            load_rows(std::true_type{}, base + NSTG * kStep, kb, blk_next);
        }
        // the tile holding the new token (fused step): its key row goes into
        // the K operand here, its value row over the staged one below
        const int dp = patch_row - base;                    // new token relative to the step
        const bool patch = FUSED && (ILV ? static_cast<unsigned>(dp) < static_cast<unsigned>(kStep) &&
                                               ((dp >> 2) & 3) == wave
                                         : static_cast<unsigned>(dp) < static_cast<unsigned>(TT));
        const int rt = ILV ? 4 * (dp >> 4) + (dp & 3) : dp;  // its row in this wave's tile
        if constexpr (FUSED) {
            if (patch) {
                // lanes of row rt % 16 of block rt / 16; every block written
                // through value selects (selecting between arrays would take
                // their addresses)
#pragma unroll
                for (int h = 0; h < KB; ++h) {
                    const bool mine = (rt >> 4) == h && r16 == (rt & 15);
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk) ka[h][kk] = select4(mine, kn[kk], ka[h][kk]);
                }
            }
        }
        // scores S^T = K Q^T, scaled to log2 units; tokens past t_end masked
        constexpr int NS = 4 * KB;            // scores per lane and head
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
                    const int t = tok(base, 16 * kb + 4 * q4 + e);
                    // (contiguous single-token splits start at t_lo)
                    const bool in = MQ ? (t >= row_lo[hb] && t < row_hi[hb])
                                       : ((PAGED ? t >= t_lo : true) && t < t_end);
                    s[hb][4 * kb + e] = in ? acc[e] * p.scale_log2 : -INFINITY;
                }
            }

        // online softmax per head.  The reference max m is only moved when the
        // tile max exceeds it by more than 2^kLazy (then O and l are rescaled);
        // otherwise p = 2^(s - m) <= 2^kLazy, exact after the final division.
        // P^T goes in as three bf16 B operands, hi + mid + lo = p to ~24
        // significant bits (the 32-row multi-token kernel, whose registers
        // have no room for a third, as two: ~16 bits).
        constexpr bool P3 = !(MQ && HB == 2);
        uint32_t ph[HB][NS / 2], pm[HB][NS / 2], pl[HB][NS / 2];
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
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[hb][nb] *= alpha;
            }
            float pr[NS], ps = 0.0f;
#pragma unroll
            for (int e = 0; e < NS; ++e) {
                pr[e] = fast_exp2(s[hb][e] - m[hb]);
                ps += pr[e];
            }
#pragma unroll
            for (int i = 0; i < NS / 2; ++i) {
                ph[hb][i] = pack2_bf16(pr[2 * i], pr[2 * i + 1]);
                const float r0 = pr[2 * i] - bf16_lo(ph[hb][i]), r1 = pr[2 * i + 1] - bf16_hi(ph[hb][i]);
                pm[hb][i] = pack2_bf16(r0, r1);
                if constexpr (P3) pl[hb][i] = pack2_bf16(r0 - bf16_lo(pm[hb][i]), r1 - bf16_hi(pm[hb][i]));
            }
            l[hb] += ps;
        }

        // This tile's V rows were issued before kAfterV later loads, and
        // loads complete in order, so waiting until at most kAfterV are
        // outstanding means they are in LDS.  The wait is explicit: the
        // compiler's own tracking of direct-to-LDS loads was seen to drop it
        // when the first tile is loaded before the loop (the transposed
        // reads then ran ahead of the data from the second iteration on).
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterV));
        if constexpr (FUSED) {
            // (every lane writes; lanes l, l + LPR, ... write the same chunk)
            if (patch) *reinterpret_cast<uint4*>(wbuf + rt * ROWB + 16 * ((lane % LPR) ^ swz(rt))) = vn;
        }

        // O^T += V^T P^T: V^T operands read transposed from LDS.  A 32-row
        // tile is one 16x16x32 product per column block (tokens of rows
        // tr_row and tr_row + 16); a 16-row tile one 16x16x16 product, whose
        // operands are exactly the low halves of those.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int u = 2 * nb + (s16 % 4) / 2;
            const int r0 = tr_row;
            const char* a0 = wbuf + r0 * ROWB + 16 * (u ^ swz(r0)) + 8 * (s16 & 1);
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a0);
            if constexpr (KB == 2) {
                const int r1 = tr_row + 16;
                const char* a1 = wbuf + r1 * ROWB + 16 * (u ^ swz(r1)) + 8 * (s16 & 1);
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a1);
                uint4 va;
                va.x = __builtin_bit_cast(uint2, lo).x;
                va.y = __builtin_bit_cast(uint2, lo).y;
                va.z = __builtin_bit_cast(uint2, hi).x;
                va.w = __builtin_bit_cast(uint2, hi).y;
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    o[hb][nb] = mfma16(va, make_uint4(ph[hb][0], ph[hb][1], ph[hb][2], ph[hb][3]), o[hb][nb]);
                    o[hb][nb] = mfma16(va, make_uint4(pm[hb][0], pm[hb][1], pm[hb][2], pm[hb][3]), o[hb][nb]);
                    if constexpr (P3)
                        o[hb][nb] = mfma16(va, make_uint4(pl[hb][0], pl[hb][1], pl[hb][2], pl[hb][3]), o[hb][nb]);
                }
            } else {
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    o[hb][nb] = mfma16k16(lo, make_uint2(ph[hb][0], ph[hb][1]), o[hb][nb]);
                    o[hb][nb] = mfma16k16(lo, make_uint2(pm[hb][0], pm[hb][1]), o[hb][nb]);
                    if constexpr (P3) o[hb][nb] = mfma16k16(lo, make_uint2(pl[hb][0], pl[hb][1]), o[hb][nb]);
                }
            }
        }
        if constexpr (KLDS) {
            // the V stage is free: the V rows of the tile NSTG steps ahead go
            // out.  (Issued before the products instead - the operand reads
            // first, then the refill, then the products behind a scheduling
            // barrier - the stream ran ~1 % slower: the products then no
            // longer overlap the transposed reads.)
            __builtin_amdgcn_s_waitcnt(kLgkmZero);
            load_rows(std::false_type{}, base + NSTG * kStep, buf, blk_next);
        }
    };

    // Software pipeline.  Staged K: the tile computation itself issues the
    // next tile's loads.  K in registers: while one tile is computed, the
    // next one's K rows and V rows (the other LDS buffer) are in flight.
    // The next tile is fetched unconditionally - past the split it reads
    // zeros (contiguous: outside the buffer range, no memory traffic) or the
    // clamped last row (paged) - so every path through the loop has the same
    // loads in flight and the waits stay exact.
    if (base < t_end) {
        if constexpr (KLDS && NSTG == 2) {
            for (;;) {
                compute_tile(ka0, kbuf, vbuf0, base);
                base += kStep;
                if (base >= t_end) break;
                compute_tile(ka0, kbuf1, vbuf1, base);
                base += kStep;
                if (base >= t_end) break;
            }
        } else if constexpr (KLDS) {
            for (;;) {
                compute_tile(ka0, kbuf, vbuf0, base);
                base += kStep;
                if (base >= t_end) break;
            }
        } else {
            auto refill = [&](int at, uint4 (&ka)[KB][KK], char* vb) __attribute__((always_inline)) {
                __builtin_amdgcn_s_waitcnt(kLgkmZero);
                load_tile(at, ka, kbuf, vb);
            };
            for (;;) {
                refill(base + kStep, ka1, vbuf1);
                compute_tile(ka0, kbuf, vbuf0, base);
                base += kStep;
                if (base >= t_end) break;
                refill(base + kStep, ka0, vbuf0);
                compute_tile(ka1, kbuf, vbuf1, base);
                base += kStep;
                if (base >= t_end) break;
            }
        }
    }

    // ---- merge the waves (LDS reused: all waves are past their loops, and
    // the last prefetch into LDS must have landed before it is overwritten)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) l[hb] = sum_same_head(l[hb]);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    if constexpr (FUSED) {
        // Results of the append: the rotated query (split 0) and the new
        // token's rotated key and raw value (the split that holds it),
        // stored once every load of this workgroup has completed.  Nothing in
        // this kernel reads them back (the holding split patched the token
        // into its tile), so they can wait until here.
        const bool qout = split == 0 && wave == 0 && p.q_rot_out != nullptr;
        const __amdgpu_buffer_rsrc_t qors =
            make_uniform_rsrc(qout ? static_cast<uint16_t*>(p.q_rot_out) + qgrp : p.q_rot_out, qout ? G * D * 2 : 0);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, qb[hb][kk]), qors,
                                                       ((16 * hb + r16) * D + 32 * kk + 8 * q4) * 2, 0, 0);
        const bool st = slot_ok && wave == 0;
        const __amdgpu_buffer_rsrc_t ksrs = make_uniform_rsrc(static_cast<const uint16_t*>(p.k) + slot, st ? D * 2 : 0);
        const __amdgpu_buffer_rsrc_t vsrs = make_uniform_rsrc(static_cast<const uint16_t*>(p.v) + slot, st ? D * 2 : 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, kn[kk]), ksrs, (32 * kk + 8 * q4) * 2, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vn), vsrs, (lane % LPR) * 16, 0, 0);
    }
    // The waves' partial results go through LDS, RB head rows at a time:
    // [NW][RB1][D] floats of O fit in one stage buffer (RB1 = 8 for 16-row
    // tiles, 16 for 32-row tiles); with K staged too, rows RB1.. go to the K
    // buffer, so a whole 16-head block takes one pass (two barriers) at
    // every tile height.  Rows are D floats apart, a multiple of the 256
    // bytes one sweep of the banks serves: the 16-byte chunks of row r are
    // XOR-swizzled by r mod 16, so the 16 lanes of one 128-bit store (one
    // column chunk of 16 rows) fill a sweep without conflicts, and 16 threads
    // reading consecutive chunks of one row do too.
    constexpr int RB1 = (STAGE / (4 * D)) < 16 ? (STAGE / (4 * D)) : 16;
    constexpr bool TWO = KLDS && RB1 < 16 && !MQ;   // (the multi-token kernel has no registers to spare)
    constexpr int RB = TWO ? 2 * RB1 : RB1;
    constexpr int NCH = D / 4;            // 16-byte chunks per row
    static_assert(NW * RB1 * D * 4 <= NW * STAGE && RB >= 4, "merge area");
    static_assert(NCH >= 16, "16 swizzle slots per row");
    auto chunk_at = [](int row, int ch) { return ch ^ (row & 15); };
    auto o_row = [&](int w, int row) __attribute__((always_inline)) {
        char* region = (TWO && row >= RB1) ? kbuf : vbuf0;
        return reinterpret_cast<float*>(region) + (w * RB1 + (TWO && row >= RB1 ? row - RB1 : row)) * D;
    };
    // (the in-kernel merge's partials: offsets below 2^31, as planned)
    const __amdgpu_buffer_rsrc_t part_rs = make_uniform_rsrc(p.ws_part, 0x7FFFFFFF);
    const __amdgpu_buffer_rsrc_t ml_rs = make_uniform_rsrc(p.ws_ml, 0x7FFFFFFF);
    float* sm_m = sm_ml;                  // [NW][16]
    float* sm_l = sm_ml + NW * 16;        // [NW][16]
    const int NT = NW * 64;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        if (q4 == 0) {
            sm_m[wave * 16 + r16] = m[hb];
            sm_l[wave * 16 + r16] = l[hb];
        }
        // query rows of this head block (MQ: of this chunk of the G * qlen rows)
        const int heads = MQ ? min(16, G * p.qlen - chunk * 16 * HB - 16 * hb) : min(16, G - 16 * hb);
        for (int r0 = 0; r0 < heads; r0 += RB) {
            // lane holds O^T[c][g] for c = 16*nb + 4*q4 + e, g = 16*hb + r16
            const int row = r16 - r0;
            if (row >= 0 && row < RB && r16 < heads) {
                float* dst = o_row(wave, row);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    *reinterpret_cast<float4*>(dst + 4 * chunk_at(row, 4 * nb + q4)) =
                        make_float4(o[hb][nb][0], o[hb][nb][1], o[hb][nb][2], o[hb][nb][3]);
            }
            __syncthreads();
            // one 16-byte column chunk of one head row per thread
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
                    const float4 ow = *reinterpret_cast<const float4*>(o_row(w, gr) + at);
                    A.x = fmaf(ow.x, f, A.x);
                    A.y = fmaf(ow.y, f, A.y);
                    A.z = fmaf(ow.z, f, A.z);
                    A.w = fmaf(ow.w, f, A.w);
                    Ls = fmaf(sm_l[w * 16 + gh], f, Ls);
                }
                size_t bh;                // output row: (b, h), or (b, i, h) for several new tokens
                if constexpr (MQ) {
                    const int rho = chunk * 16 * HB + 16 * hb + gh;
                    const int qi = rho / G;
                    bh = (static_cast<size_t>(b) * p.qlen + qi) * p.H_q + j * G + (rho - qi * G);
                } else {
                    bh = static_cast<size_t>(b) * p.H_q + j * G + 16 * hb + gh;
                }
                const int c = 4 * ch;
                if (nsp == 1) {
                    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
                    uint2 packed;
                    packed.x = static_cast<uint32_t>(f32_to_bf16_rne(A.x * inv)) |
                               (static_cast<uint32_t>(f32_to_bf16_rne(A.y * inv)) << 16);
                    packed.y = static_cast<uint32_t>(f32_to_bf16_rne(A.z * inv)) |
                               (static_cast<uint32_t>(f32_to_bf16_rne(A.w * inv)) << 16);
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

    // ---- merge of the unit's splits by the last of them to finish.  The
    // partial rows above went out as device-scope stores; once they have
    // completed, each split counts itself in.  The increment wraps at
    // nsp - 1, so the split that reads nsp - 1 is the last (it leaves the
    // counter at zero for the next call) and reads every split's rows back
    // with device-scope loads.  No workgroup ever waits for another, and no
    // cache is flushed.  The merge: M = max_s m_s, w_s = 2^(m_s - M),
    // out = sum_s w_s acc_s / sum_s w_s l_s, the splits in order, MB of them
    // requested at a time (their max folded into the running one).
    // (Balanced schedule: the unit's partials are those of workgroups wf ..
    // wf + nsp - 1, each in its first-segment slot except maybe the first's.)
    if (nsp > 1 && p.merge_cnt != nullptr) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        if (tid == 0)
            s_last = __builtin_amdgcn_atomic_inc32(p.merge_cnt + unit, static_cast<unsigned>(nsp - 1),
                                                   __ATOMIC_RELAXED, "agent") == static_cast<unsigned>(nsp - 1);
        __syncthreads();
        if (!s_last) continue;
        const int rows = MQ ? min(16 * HB, G * p.qlen - chunk * 16 * HB) : G;
        auto row_of = [&](int gr) -> size_t {
            if constexpr (MQ) {
                const int rho = chunk * 16 * HB + gr;
                const int qi = rho / G;
                return (static_cast<size_t>(b) * p.qlen + qi) * p.H_q + j * G + (rho - qi * G);
            } else {
                return static_cast<size_t>(b) * p.H_q + j * G + gr;
            }
        };
        merge_split_rows<D>(p, part_rs, ml_rs, rows, nsp, row_of, [&](int gr, int sp) -> size_t {
            if constexpr (BAL)
                return bal_part_row(p, sg, gr, sp);
            else
                return row_of(gr) * p.n_splits + sp;
        });
    }
    }   // segments
}

constexpr int kNWm = 4;

template <int D, int HB, bool FUSED, bool MQ>
hipError_t launch_dhf(bool paged, const DecodeParams& p, hipStream_t stream, const KernelTiming& tm) {
    const dim3 grid(p.n_wg_pad), block(kNWm * 64);
    const int32_t* tbl = p.block_table;
    if constexpr (D <= 128 && !MQ) {
        // balanced schedule (planned for paged pools, d <= 128, one new token,
        // no window, block sizes that are multiples of 16, at most kBalMaxB
        // sequences)
        if (p.bal) {
            if (!paged || p.B > kBalMaxB || p.block_size % 16 != 0) return hipErrorInvalidValue;
            return launch_timed(decode_mfma_kernel<D, HB, kNWm, 3, FUSED, MQ, true>, grid, block, stream, tm, p, tbl);
        }
    }
    if (p.bal) return hipErrorInvalidValue;
    if (!paged)
        return launch_timed(decode_mfma_kernel<D, HB, kNWm, 0, FUSED, MQ, false>, grid, block, stream, tm, p, tbl);
    if constexpr (D <= 128) {
        if (p.block_size % 16 == 0 && p.split_tokens % 16 == 0 && p.split_tokens / p.block_size + 2 <= kTblMax)
            return launch_timed(decode_mfma_kernel<D, HB, kNWm, 3, FUSED, MQ, false>, grid, block, stream, tm, p,
                                tbl);
    }
    if (p.block_size % 16 == 0 && p.split_tokens % 32 == 0)
        return launch_timed(decode_mfma_kernel<D, HB, kNWm, 2, FUSED, MQ, false>, grid, block, stream, tm, p, tbl);
    return launch_timed(decode_mfma_kernel<D, HB, kNWm, 1, FUSED, MQ, false>, grid, block, stream, tm, p, tbl);
}

// rows: query rows one workgroup serves (G, or a chunk of the G * qlen rows
// of several new tokens), in one or two 16-row head blocks
template <int D>
hipError_t launch_d(int rows, bool paged, bool fused, bool multi, const DecodeParams& p, hipStream_t stream,
                    const KernelTiming& tm) {
    if (multi)
        return rows <= 16 ? launch_dhf<D, 1, false, true>(paged, p, stream, tm)
                          : launch_dhf<D, 2, false, true>(paged, p, stream, tm);
    if (rows <= 16)
        return fused ? launch_dhf<D, 1, true, false>(paged, p, stream, tm)
                     : launch_dhf<D, 1, false, false>(paged, p, stream, tm);
    return fused ? launch_dhf<D, 2, true, false>(paged, p, stream, tm)
                 : launch_dhf<D, 2, false, false>(paged, p, stream, tm);
}

}  // namespace

bool decode_mfma_supported(kvc_dtype dtype, int d, int G) {
    return dtype == KVC_BF16 && (d == 64 || d == 128 || d == 256) && G >= 1 && G <= 32;
}

int decode_mfma_step_tokens(int d, bool /*paged*/) { return kNWm * (d <= 128 ? 16 : 32); }

int decode_mfma_wgs_per_cu(int d, int G, bool paged) {
    // Per workgroup: 4 waves; LDS TT * 2d bytes per staged tile.  Up to
    // d = 128 (TT = 16): one K and one V tile per wave, 16 KiB at d = 64 and
    // 32 KiB at d = 128, plus 4 KiB of block table when paged.  A contiguous
    // cache at d = 128 still streamed best with one workgroup per CU (its
    // 32 KiB in flight is what a plain streaming read needs; two measured
    // about 1.5 % slower); a ragged paged pool, whose many short splits each
    // pay a prologue, with three (registers: at most 168 per lane with one
    // 16-head block, three waves per SIMD).  Two 16-head blocks: planned as
    // one, though over a contiguous cache the kernel's registers are held to
    // two waves per SIMD and a CU runs two of them (the split plans for those
    // groups, about three workgroups per slot, were measured with this count:
    // doubling it doubled the multi-token workload's splits, 96 -> 106 us).
    // At d = 256 (TT = 32, K in registers): two V tiles per wave, 128 KiB.
    const bool two_blocks = G > 16;
    if (d <= 64) return two_blocks ? 2 : (paged ? 3 : 2);
    if (d <= 128) return two_blocks ? 1 : (paged ? 3 : 1);
    return 1;
}

hipError_t launch_decode_mfma(int d, int rows, bool paged, bool fused, bool multi, const DecodeParams& p,
                              hipStream_t stream, const KernelTiming& tm) {
    switch (d) {
        case 64: return launch_d<64>(rows, paged, fused, multi, p, stream, tm);
        case 128: return launch_d<128>(rows, paged, fused, multi, p, stream, tm);
        case 256: return launch_d<256>(rows, paged, fused, multi, p, stream, tm);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
