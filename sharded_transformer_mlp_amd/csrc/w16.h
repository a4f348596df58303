// Shape-6 MFMA pipeline (gfx950), shared by the forward kernels and the
// backward's matrix products.
//
// A 256 x 256 output tile per workgroup, 4 waves (one per SIMD) as 2 x 2, each
// wave a 128 x 128 piece held in 64 16x16 fp32 accumulators (all 256
// accumulation registers), v_mfma_f32_16x16x32_bf16. Operands stream through
// a 5-stage LDS ring of 32-deep reduction stages (5 x 32 KiB = all 160 KiB)
// filled by global-to-LDS loads; a wave reads 16 fragments per 64 MFMAs.
//
// The first reduction step starts every accumulator from the constant 0
// (MFMA source C = 0) instead of adding to zero-initialised registers: with
// that form the compiler keeps each accumulator in one register across the
// loop (with zero-initialised registers it copies accumulators between
// registers on every trip).
//
// An operand source (Src) supplies one stage's loads for this wave, the
// fragment reads, and the walk over the reduction dimension:
//   void issue(int g, uint16_t* lds_stage)   load g of LOADS for the current stage
//   void advance()                           next stage (clamped to the last one)
//   void read(int q, const uint16_t* lds_stage, bf16x8 (&af)[TM], bf16x8 (&bv)[TN])
// PackedSrc takes the A operand from packed 32 x 16 fragment blocks (the
// forward's weight records); RowSrc takes it from a row-major matrix with
// the reduction index contiguous, like the B operand (the backward).
#pragma once

#include "common.h"

namespace tsp {

// Fourth word of a raw (untyped, unswizzled) buffer resource on this GPU
// family: 32-bit data format, no index stride.
constexpr int kRawBufferWord3 = 0x00020000;

// LDS slot of row r's 8-index chunk c in a 16-row x 32-index operand block
// (1 KiB). The 16x16x32 fragment read has lane l take row l % 16, chunk
// l / 16; with this XOR (on r / 2) that read runs without LDS bank conflicts
// (measured with SQ_LDS_BANK_CONFLICT; an XOR on r / 4 costs it a 2-way
// conflict). Each group of 4 lanes still loads the 64 contiguous bytes of
// one row.
__device__ __forceinline__ int b_slot(int r, int c) { return 4 * r + (c ^ ((r >> 1) & 3)); }

namespace w16 {

constexpr int BM = 256, BN = 256, NW = 4, WN = 2;
constexpr int TM = 8, TN = 8;                           // 16-row / 16-token MFMA blocks per wave
constexpr int A_BLK = BM / 16, B_BLK = BN / 16;         // 1 KiB blocks per 32-wide stage
constexpr int LA = A_BLK / NW, LB = B_BLK / NW;         // blocks each wave loads per stage
constexpr int LOADS = LA + LB;
constexpr int STAGE = (A_BLK + B_BLK) * 512;
constexpr int NS = 5;                                   // 5 x 32 KiB = all 160 KiB of LDS
static_assert(NS * STAGE * 2 <= 160 * 1024, "LDS");
static_assert((NS - 1) * LOADS <= 63, "vmcnt range");

#define TSP_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// One 16-row x 32-index block of a row-major operand into LDS: lane l loads
// row row0 + l / 4 (clamped to last_row) and the 16 bytes that land in slot
// l, i.e. chunk (l % 4) ^ ((l / 8) % 4) of that row's 64 bytes at base + row *
// ld (base already at the stage's reduction offset). BUF: buffer load with a
// 32-bit offset from base (the caller keeps every offset below 2^31 bytes).
template <bool BUF>
__device__ __forceinline__ void load_rows(uint16_t* lds_blk, const uint16_t* __restrict__ base, int ld, int row0,
                                          int last_row, int lane) {
    const int rr = lane >> 2;
    const int c = (lane & 3) ^ ((rr >> 1) & 3);         // slot = lane = b_slot(rr, c)
    TSP_LDS void* dst = (TSP_LDS void*)lds_blk;
    const int row = min(row0 + rr, last_row);
    const int64_t off = (int64_t)row * ld + c * 8;
    if constexpr (BUF) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, kRawBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (int)(off * 2), 0, 0, 0);
    } else {
        __builtin_amdgcn_global_load_lds(base + off, dst, 16, 0, 0);
    }
}

// Fragment q of a row-block region: rows 16 q' + l % 16, chunk l / 16.
__device__ __forceinline__ bf16x8 read_rows(const uint16_t* region, int blk, int lane) {
    const int r = lane & 15, c = lane >> 4;
    return reinterpret_cast<const bf16x8*>(region)[blk * 64 + b_slot(r, c)];
}

// Forward operands: A = packed weight records (32 x 16 fragment blocks, a
// stage's 256 rows are 8 blocks of 32 rows, each two 1 KiB blocks deep), B =
// token rows (T x ldb row-major). spp > 0 (down product): the reduction walks
// shard records, spp steps each, a_rec elements apart.
template <bool BUF>
struct PackedSrc {
    const uint16_t* a;                                  // A slab of the current stage
    int tl, ls;                                         // stage index, step inside the record
    int ksteps, spp;
    int64_t a_rec, a_rs;                                // record stride, 32-row block stride (elements)
    const uint16_t* b_src;
    int ldb, t0, T, w, wm, wn, lane;

    __device__ void issue(int g, uint16_t* lds_stage) {
        if (g < LA) {
            const int b = g * NW + w;
            TSP_LDS void* dst = (TSP_LDS void*)(lds_stage + b * 512);
            const int64_t off = (b >> 1) * a_rs + (b & 1) * 512 + lane * 8;
            if constexpr (BUF) {
                const __amdgpu_buffer_rsrc_t rs =
                    __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, 0x7fffffff, kRawBufferWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (int)(off * 2), 0, 0, 0);
            } else {
                __builtin_amdgcn_global_load_lds(a + off, dst, 16, 0, 0);
            }
        } else {
            const int bb = (g - LA) * NW + w;
            load_rows<BUF>(lds_stage + (A_BLK + bb) * 512, b_src + (int64_t)tl * 32, ldb, t0 + bb * 16, T - 1, lane);
        }
    }
    __device__ void advance() {
        const bool adv = tl + 1 < ksteps;
        const bool wrap = spp > 0 && ls + 1 == spp;
        a += adv ? (wrap ? a_rec - (int64_t)(spp - 1) * 1024 : (int64_t)1024) : (int64_t)0;
        ls = adv ? (wrap ? 0 : ls + 1) : ls;
        tl += adv ? 1 : 0;
    }
    // A fragment q: 16-row block ib = rows 16 (ib % 2) + l % 16 of 32-row block
    // ib / 2, reduction indices 8 (l / 16) .. + 7 (two 1 KiB blocks deep).
    __device__ void read(int q, const uint16_t* lds_stage, bf16x8 (&af)[TM], bf16x8 (&bv)[TN]) const {
        if (q < TM) {
            const int r = lane & 15, c = lane >> 4;
            const bf16x8* as = reinterpret_cast<const bf16x8*>(lds_stage);
            const int ib = wm * TM + q;
            af[q] = as[((ib >> 1) * 2 + (c >> 1)) * 64 + (c & 1) * 32 + (ib & 1) * 16 + r];
        } else {
            bv[q - TM] = read_rows(lds_stage + A_BLK * 512, wn * TN + q - TM, lane);
        }
    }
};

// Backward operands: C[n][m] = sum_k A[m][k] B[n][k] with A (M x K, lda) and
// B (N x K, ldb) row-major, both loaded like the forward's token operand. The
// reduction runs over nseg segments of spp steps; segment j uses A and B at
// a_base[j % kinds] + (order ? order[j / kinds] : j / kinds) * a_seg and
// b_base[j % kinds] + (j / kinds) * b_seg (elements along the rows), which
// walks (gate, up) column blocks of the weights in ring order for dX.
template <bool BUF>
struct RowSrc {
    const uint16_t* a;                                  // A at the current stage's reduction offset
    const uint16_t* b;
    int ls, j;                                          // step inside the segment, segment
    int spp, nseg, kinds;
    const uint16_t *a_base0, *a_base1;                  // segment kinds 0 and 1 (no indexed arrays:
    const uint16_t *b_base0, *b_base1;                  // a runtime index would put them in scratch)
    int64_t a_seg, b_seg;
    const int32_t* order;
    int lda, ldb, m0, n0, last_m, last_n, w, wm, wn, lane;

    __device__ void seek(int seg) {
        const int kind = seg % kinds, k = seg / kinds;
        // wave-uniform (the buffer resource built from it must live in SGPRs)
        const int s = order ? __builtin_amdgcn_readfirstlane(order[k]) : k;
        a = (kind ? a_base1 : a_base0) + (int64_t)s * a_seg;
        b = (kind ? b_base1 : b_base0) + (int64_t)k * b_seg;
    }
    __device__ void issue(int g, uint16_t* lds_stage) {
        if (g < LA) {
            const int blk = g * NW + w;
            load_rows<BUF>(lds_stage + blk * 512, a, lda, m0 + blk * 16, last_m, lane);
        } else {
            const int bb = (g - LA) * NW + w;
            load_rows<BUF>(lds_stage + (A_BLK + bb) * 512, b, ldb, n0 + bb * 16, last_n, lane);
        }
    }
    __device__ void advance() {
        if (ls + 1 < spp) {
            ++ls;
            a += 32;
            b += 32;
        } else if (j + 1 < nseg) {
            ls = 0;
            seek(++j);
        }
    }
    __device__ void read(int q, const uint16_t* lds_stage, bf16x8 (&af)[TM], bf16x8 (&bv)[TN]) const {
        if (q < TM) af[q] = read_rows(lds_stage, wm * TM + q, lane);
        else bv[q - TM] = read_rows(lds_stage + A_BLK * 512, wn * TN + q - TM, lane);
    }
};

__device__ __forceinline__ int next_buf(int off) { return off == (NS - 1) * STAGE ? 0 : off + STAGE; }

// Step t. The barrier makes every wave's share of stage t + 1 visible and
// ends every wave's fragment reads of stage t (issued in step t - 1), so
// stage t's buffer takes the loads of stage t + NS. The wave then reads stage
// t + 1's fragments into the other register set while its MFMAs run on stage
// t's, and before the next barrier waits for those reads and for its own
// loads of stage t + 2. Every step issues one stage (past the end, the last
// stage again, into a buffer nobody reads), so that wait is always "at most 3
// stages newer". FIRST: the accumulators start from 0. LAST: MFMAs only.
//
// With one wave per SIMD nothing else feeds the matrix pipe while this wave
// issues other work, so scheduling fences fix the order: three MFMAs right
// after the barrier, then eight groups of one load, two fragment reads and
// seven MFMAs (a load right after another costs the matrix pipe far more
// than one that follows a few MFMAs: 3-5 % of the kernel time here), and the
// scalar bookkeeping for the next step spread over the last five MFMAs.
template <bool FIRST, bool LAST, class Src>
__device__ __forceinline__ void step(int& ld_ref, int& rd_ref, Src& src, uint16_t* lds, f32x4 (&acc)[TM][TN],
                                     const bf16x8 (&ca)[TM], const bf16x8 (&cb)[TN], bf16x8 (&na)[TM],
                                     bf16x8 (&nb)[TN]) {
    constexpr int LEAD = 3, GROUP = 7;
    constexpr int TAIL = TM * TN - LEAD - LOADS * GROUP;
    static_assert(LOADS == 8 && TM + TN == 2 * LOADS && TAIL == 5, "schedule");
    auto mf = [&](int m) {
        const int i = m / TN, j = m % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[i], cb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f}
                                                                                : acc[i][j], 0, 0, 0);
    };
    if constexpr (LAST) {
#pragma unroll
        for (int m = 0; m < TM * TN; ++m) mf(m);
        return;
    }
    const int ld_off = ld_ref, rd_off = rd_ref;
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < LEAD; ++m) mf(m);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < LOADS; ++g) {
        const int m0 = LEAD + GROUP * g;
        src.issue(g, lds + ld_off);
        mf(m0);
        mf(m0 + 1);
        __builtin_amdgcn_sched_barrier(0);
        src.read(2 * g, lds + rd_off, na, nb);
        mf(m0 + 2);
        mf(m0 + 3);
        __builtin_amdgcn_sched_barrier(0);
        src.read(2 * g + 1, lds + rd_off, na, nb);
        mf(m0 + 4);
        mf(m0 + 5);
        mf(m0 + 6);
        __builtin_amdgcn_sched_barrier(0);
    }
    src.advance();
    ld_ref = rd_off;
    rd_ref = next_buf(rd_off);
#pragma unroll
    for (int m = TM * TN - TAIL; m < TM * TN; ++m) mf(m);
#pragma unroll
    for (int k = 0; k < TAIL; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x006, 4, 0);   // VALU / SALU
    }
    __builtin_amdgcn_sched_barrier(0);
    TSP_VMCNT(3 * LOADS);                               // own loads of stage t + 2 landed
    lgkm_zero();                                        // stage t + 1's fragments in registers
    __builtin_amdgcn_sched_barrier(0);
}

// One stream of stages through the LDS ring. start() issues the first NS
// stages and reads stage 0's fragments; tile() runs one tile's ksteps stages
// (even, >= 2) from the stream, leaving the next tile's stage-0 fragments in
// (a0, b0) unless END; finish() waits for every load into LDS. A workgroup
// that runs several tiles back to back (a source whose advance() walks on to
// the next tile) thus issues the next tile's first loads during this tile's
// last steps, and they land while it writes its results.
template <class Src>
struct Stream {
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    int ld = 0, rd = STAGE;                             // buffers of stages t and t + 1

    __device__ __forceinline__ void start(uint16_t* lds, Src& src) {
        for (int t = 0; t < NS; ++t) {
#pragma unroll
            for (int g = 0; g < LOADS; ++g) src.issue(g, lds + t * STAGE);
            src.advance();
        }
        TSP_VMCNT((NS - 1) * LOADS);                    // own loads of stage 0 landed
        stage_barrier();
#pragma unroll
        for (int q = 0; q < TM + TN; ++q) src.read(q, lds, a0, b0);
        TSP_VMCNT((NS - 2) * LOADS);                    // own loads of stage 1 landed
        lgkm_zero();
        __builtin_amdgcn_sched_barrier(0);
    }
    template <bool END>
    __device__ __forceinline__ void tile(uint16_t* lds, f32x4 (&acc)[TM][TN], int ksteps, Src& src) {
        step<true, false>(ld, rd, src, lds, acc, a0, b0, a1, b1);
        for (int t = 1; t + 2 < ksteps; t += 2) {
            step<false, false>(ld, rd, src, lds, acc, a1, b1, a0, b0);
            step<false, false>(ld, rd, src, lds, acc, a0, b0, a1, b1);
        }
        step<false, END>(ld, rd, src, lds, acc, a1, b1, a0, b0);
    }
    __device__ __forceinline__ void finish() {
        TSP_VMCNT(0);                                   // no load into LDS outlives the workgroup
    }
};

// A workgroup's bf16 result rows staged in the LDS ring once the reduction is
// done, so that the global stores write whole rows: straight from the MFMA
// layout, a store covers 16 tokens x 32 bytes, a quarter of a 128-byte line per
// token (measured: 17 % of the backward gate/up kernel's time went to three
// such stores). ROWS = 256 stages the whole token tile; ROWS = 128 stages one
// half hh of each wave row's 128 tokens (tile rows wn * 128 + hh * 64 + [0, 64)
// at staged rows wn * 64 + [0, 64)), for epilogues with more outputs than the
// ring holds at full height. put4 takes one lane's four values at a staged row;
// the row pitch COLS + 8 spreads a put4 instruction's 16 rows over all banks.
// flush() writes the staged rows of this wave's quarter.
template <int COLS, int ROWS = 256>
struct StagedRows16 {
    static_assert(ROWS == 256 || ROWS == 128, "ROWS");
    static constexpr int PITCH = COLS + 8;
    static constexpr int ELEMS = ROWS * PITCH;          // LDS elements one staged tile takes
    static_assert(ELEMS * 2 <= NS * STAGE * 2, "LDS");
    uint16_t* lds;
    __device__ __forceinline__ void put4(int r, int c, uint2 v) {
        *reinterpret_cast<uint2*>(lds + r * PITCH + c) = v;
    }
    __device__ __forceinline__ void flush(uint16_t* __restrict__ dst, int64_t ld, int t0, int T, int64_t col0,
                                          int w, int lane, int hh = 0) {
        constexpr int LPR = COLS / 8;                   // lanes per row (16 bytes each)
        constexpr int RPI = 64 / LPR;                   // rows per store instruction
        constexpr int RPW = ROWS / 4;                   // staged rows per wave
#pragma unroll
        for (int it = 0; it < RPW / RPI; ++it) {
            const int r = w * RPW + it * RPI + lane / LPR;
            const int c = (lane % LPR) * 8;
            const int tr = ROWS == 256 ? r : (r >> 6) * 128 + hh * 64 + (r & 63);
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * PITCH + c);
            if (t0 + tr < T) *reinterpret_cast<u32x4*>(dst + (int64_t)(t0 + tr) * ld + col0 + c) = v;
        }
    }
};

// The fp32 counterpart for 256-column result tiles: 128 staged rows, one half
// hh of each wave row's tokens (as StagedRows16<COLS, 128>), 1 KiB per row so
// that each flush store writes one whole row. put4 takes one lane's four
// values; the pitch 260 puts a put4 instruction's 16 rows 4 banks apart.
struct StagedRowsF32 {
    static constexpr int COLS = 256, ROWS = 128, PITCH = COLS + 4;
    static constexpr int ELEMS = ROWS * PITCH;          // floats
    static_assert(ELEMS * 4 <= NS * STAGE * 2, "LDS");
    float* lds;
    __device__ __forceinline__ void put4(int r, int c, f32x4 v) {
        *reinterpret_cast<f32x4*>(lds + r * PITCH + c) = v;
    }
    // rows n0 + tr + row_shift of dst for tile rows tr of half hh below N
    __device__ __forceinline__ void flush(float* __restrict__ dst, int64_t ld, int n0, int N, int64_t row_shift,
                                          int64_t col0, int w, int lane, int hh) {
#pragma unroll 8
        for (int it = 0; it < ROWS / 4; ++it) {
            const int r = w * (ROWS / 4) + it;
            const int tr = (r >> 6) * 128 + hh * 64 + (r & 63);
            const f32x4 v = *reinterpret_cast<const f32x4*>(lds + r * PITCH + lane * 4);
            if (n0 + tr < N) *reinterpret_cast<f32x4*>(dst + (n0 + tr + row_shift) * ld + col0 + lane * 4) = v;
        }
    }
};

// The reduction over ksteps stages (even, >= 2). src is positioned at stage 0.
template <class Src>
__device__ __forceinline__ void mainloop(uint16_t* lds, f32x4 (&acc)[TM][TN], int ksteps, Src& src) {
    Stream<Src> st;
    st.start(lds, src);
    st.template tile<true>(lds, acc, ksteps, src);
    st.finish();
}
#undef TSP_VMCNT

}  // namespace w16
}  // namespace tsp
