// The 256 x 256 MFMA pipeline (gfx950), shared by the forward kernels, the
// attention projection and the backward's matrix products.
//
// A 256 x 256 output tile per workgroup, 4 waves (one per SIMD) as 2 x 2, each
// wave a 128 x 128 piece held in 64 16x16 fp32 accumulators (all 256
// accumulation registers), v_mfma_f32_16x16x32_bf16, 32 reduction indices per
// step; a wave reads 16 fragments per 64 MFMAs. Operands reach LDS by
// global-to-LDS loads, in one of two rings over the 160 KiB:
//
// * the split ring (mainloop): the A operand through 4 stages 32 deep, the B
//   operand (token rows) through 3 super-stages 64 deep, so that every B load
//   instruction reads 8 whole 128-byte rows. With 64-byte row pieces each
//   instruction makes 16 cache-line requests instead of 8, and the texture
//   address unit spent a quarter of the gate/up kernel's cycles stalled on the
//   L1 (TA_ADDR_STALLED_BY_TC_CYCLES 0.31 per CU-cycle; 0.04 here). A load has
//   two steps to land.
// * the 5-stage ring (mainloop5): both operands in 32-deep stages (B in 64-byte
//   row pieces); a load has three steps to land. The down product, whose
//   operands stream from beyond the L2, runs faster on it.
//
// A step's 64 MFMAs keep one A fragment for 8 consecutive MFMAs and walk the
// B fragments in snake order (forward on even A rows, backward on odd), so
// that the B operand stays the same across each change of A: under the
// power limit fewer operand changes ran the Llama-shape forward 0.3 % faster
// (same box, bitwise equal; the A-inner order ran 0.7 % slower).
//
// The first reduction step starts every accumulator from the constant 0
// (MFMA source C = 0) instead of adding to zero-initialised registers: with
// that form the compiler keeps each accumulator in one register across the
// loop (with zero-initialised registers it copies accumulators between
// registers on every trip).
//
// PackedSrc takes the A operand from packed 32 x 16 fragment blocks (the
// forward's weight records); RowSrc (the backward) walks reduction segments
// and takes A either from a row-major matrix with the reduction index
// contiguous or (FRAG) from the same fragment-block layout. B is always
// row-major.
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

// A wave-uniform pointer kept in scalar registers (a buffer resource built
// from it must live in SGPRs; without this the compiler can lose track of
// its uniformity and wrap the load in a loop over lanes).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

constexpr int BM = 256, BN = 256, NW = 4, WN = 2;
constexpr int TM = 8, TN = 8;                           // 16-row / 16-token MFMA blocks per wave
// A operand: a ring of NA stages, 32 reduction indices each, sixteen 1 KiB
// blocks per stage (A_BLK), each wave loading LA of them per step.
constexpr int A_BLK = BM / 16;
constexpr int LA = A_BLK / NW;
constexpr int A_STAGE = A_BLK * 512;                    // elements
constexpr int NA = 4;
// B operand (token rows): a ring of NB super-stages of 64 reduction indices,
// so that every load instruction fetches 8 whole 128-byte rows (one full
// cache line per row). A super-stage is loaded in two halves of 128 rows,
// one half per step, each wave loading LB pieces of 8 rows per half.
constexpr int B_SUPER = BN * 64;                        // elements
constexpr int NB = 3;
constexpr int LB = BN / 2 / 8 / NW;
constexpr int LOADS = LA + LB;
constexpr int B_OFF = NA * A_STAGE;                     // element offset of the B ring
constexpr int LDS_ELEMS = NA * A_STAGE + NB * B_SUPER;  // 64 + 96 KiB = all 160 KiB of LDS
static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS");
static_assert(LOADS == 8, "schedule");

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

// B super-stage layout: row r's 16-byte chunk c (c = 0..7, reduction indices
// 8 c .. 8 c + 7 of the 64) sits in slot 8 r + (c ^ (r % 8)). A fragment
// read (lane l: row l % 16 of a 16-row block, chunk 4 h + l / 16 for the
// step's half h) then puts eight consecutive lanes on eight different 16-byte
// bank groups.
__device__ __forceinline__ int b64_slot(int r, int c) { return 8 * r + (c ^ (r & 7)); }

// 8 rows x 128 bytes into one 1 KiB piece of a B super-stage: lane l loads
// row row0 + l / 8 (clamped to last_row; row0 % 8 == 0) and the 16 bytes that
// land in slot l % 8 of that row, i.e. chunk (l % 8) ^ (l / 8). Every lane
// group of 8 reads one whole 128-byte row.
template <bool BUF>
__device__ __forceinline__ void load_rows128(uint16_t* lds_piece, const uint16_t* __restrict__ base, int ld,
                                             int row0, int last_row, int lane) {
    const int rr = lane >> 3;
    const int c = (lane & 7) ^ rr;                      // slot = lane = b64_slot(rr, c) - 8 rr + 8 rr
    TSP_LDS void* dst = (TSP_LDS void*)lds_piece;
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

// B fragment of 16-row block blk for the step's half h of a super-stage.
__device__ __forceinline__ bf16x8 read_rows128(const uint16_t* super, int blk, int h, int lane) {
    const int r = blk * 16 + (lane & 15), c = 4 * h + (lane >> 4);
    return reinterpret_cast<const bf16x8*>(super)[b64_slot(r, c)];
}

// An operand source supplies, for this wave:
//   issue_a(g, lds_stage)       A load g (< LA) of the current A stage
//   advance_a()                 next A stage (clamped to the last one)
//   issue_b(g, lds_super, h)    B load g (< LB) of half h of the current super-stage
//   advance_b()                 next super-stage (clamped to the last one)
//   read_a(q, lds_stage, af)    A fragment q (< TM)
// The B fragments are read by the pipeline itself (read_rows128): B is always
// a row-major token-like operand, rows b_row0 + ..., with the reduction index
// contiguous.
//
// Forward operands: A = packed weight records (32 x 16 fragment blocks, a
// stage's 256 rows are 8 blocks of 32 rows, each two 1 KiB blocks deep), B =
// token rows (T x ldb row-major). spp > 0 (down product): the reduction walks
// shard records, spp steps each, a_rec elements apart.
template <bool BUF, bool BLK = false>
struct PackedSrc {
    const uint16_t* a;                                  // A slab of the current stage
    int tl, ls;                                         // A stage index, step inside the record
    int ksteps, spp;
    int64_t a_rec, a_rs;                                // record stride, 32-row block stride (elements)
    const uint16_t* b_src;
    int ldb, t0, T, w, wm, wn, lane;
    int sb = 0;                                         // B super-stage index

    __device__ void issue_a(int g, uint16_t* lds_stage) {
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
    }
    __device__ void advance_a() {
        const bool adv = tl + 1 < ksteps;
        const bool wrap = spp > 0 && ls + 1 == spp;
        a += adv ? (wrap ? a_rec - (int64_t)(spp - 1) * 1024 : (int64_t)1024) : (int64_t)0;
        ls = adv ? (wrap ? 0 : ls + 1) : ls;
        tl += adv ? 1 : 0;
        if constexpr (BLK) bstage += adv ? bstride : (int64_t)0;
    }
    __device__ void issue_b(int g, uint16_t* lds_super, int h) {
        const int r0 = h * (BN / 2) + (g * NW + w) * 8;
        load_rows128<BUF>(lds_super + r0 * 64, b_src + (int64_t)sb * 64, ldb, t0 + r0, T - 1, lane);
    }
    __device__ void advance_b() { sb += 2 * (sb + 1) < ksteps ? 1 : 0; }
    __device__ void advance5() { advance_a(); }        // the 5-stage ring: B follows A's stage index
    int nbt = 0;                                        // BLK: 16-token blocks per 32-column block
    const uint16_t* bstage = nullptr;                   // BLK: the current stage's column block of B
    int64_t bstride = 0;                                // BLK: elements per column block
    __device__ void set_blocked(int n) {
        nbt = n;
        bstage = b_src;
        bstride = (int64_t)n * 512;
    }
    // 32-deep B stages of the 5-stage ring (mainloop5), at the A stage's
    // reduction offset (the two operands advance together there, advance_a
    // moves both): 16-row x 64-byte pieces of row-major B, or (BLK) B stored
    // in 16-token x 32-column blocks of 1 KiB (see Bf16Args::nbt), one
    // contiguous block per load; token blocks past the last are clamped to it
    // (their rows belong to tokens >= T, never stored)
    __device__ void issue_b32(int g, uint16_t* lds_blocks) {
        const int bb = g * NW + w;
        if constexpr (BLK) {
            const int tb = min((t0 >> 4) + bb, nbt - 1);
            const int rr = lane >> 2, c = (lane & 3) ^ ((rr >> 1) & 3);   // slot = lane = b_slot(rr, c)
            TSP_LDS void* dst = (TSP_LDS void*)(lds_blocks + bb * 512);
            if constexpr (BUF) {
                // the stage's column block as the resource base, the token
                // block (wave-uniform, fixed across steps) as the scalar offset:
                // no 64-bit address arithmetic per load
                const __amdgpu_buffer_rsrc_t rs =
                    __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(bstage), (short)0, 0x7fffffff, kRawBufferWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (rr * 4 + c) * 16, tb * 1024, 0, 0);
            } else {
                __builtin_amdgcn_global_load_lds(bstage + (int64_t)tb * 512 + (rr * 4 + c) * 8, dst, 16, 0, 0);
            }
        } else {
            load_rows<BUF>(lds_blocks + bb * 512, b_src + (int64_t)tl * 32, ldb, t0 + bb * 16, T - 1, lane);
        }
    }
    // A fragment q: 16-row block ib = rows 16 (ib % 2) + l % 16 of 32-row block
    // ib / 2, reduction indices 8 (l / 16) .. + 7 (two 1 KiB blocks deep).
    __device__ void read_a(int q, const uint16_t* lds_stage, bf16x8 (&af)[TM]) const {
        const int r = lane & 15, c = lane >> 4;
        const bf16x8* as = reinterpret_cast<const bf16x8*>(lds_stage);
        const int ib = wm * TM + q;
        af[q] = as[((ib >> 1) * 2 + (c >> 1)) * 64 + (c & 1) * 32 + (ib & 1) * 16 + r];
    }
};

// Backward operands: C[n][m] = sum_k A[m][k] B[n][k] with A (M x K, lda) and
// B (N x K, ldb) row-major. The reduction runs over nseg segments of spp steps;
// segment j uses A and B at a_base[j % kinds] + (order ? order[j / kinds] :
// j / kinds) * a_seg and b_base[j % kinds] + (j / kinds) * b_seg (elements
// along the rows), which walks (gate, up) column blocks of the weights in
// ring order for dX. A is loaded in 64-byte row pieces into the A ring, B in
// whole 128-byte rows into the B ring; the two walk the segments with cursors
// of their own (B runs ahead of A). spp is even.
//
// FRAG: A is stored in 32 x 16 fragment blocks (the layout of the packed
// weight records, rows = m, reduction index = k, K = lda: block (m / 32,
// k / 16) at element ((m / 32) (lda / 16) + k / 16) 512, lane l of a block
// holding row l % 32 and indices 8 (l / 32) .. + 7). A stage's A loads are
// then whole 1 KiB blocks (8 cache lines per load instruction instead of the
// 16 that 64-byte row pieces touch), as for the forward's weights. Offsets
// along the rows (a_seg, the 32-index steps) keep their row-major meaning and
// become 32x as many elements.
template <bool BUF, bool FRAG = false>
struct RowSrc {
    const uint16_t* a;                                  // A at the current stage's reduction offset
    const uint16_t* b;                                  // B at the current super-stage's offset
    int ls, j;                                          // A: step inside the segment, segment
    int lsb, jb;                                        // B: super-stage inside the segment, segment
    int spp, nseg, kinds;
    const uint16_t *a_base0, *a_base1;                  // segment kinds 0 and 1 (no indexed arrays:
    const uint16_t *b_base0, *b_base1;                  // a runtime index would put them in scratch)
    int64_t a_seg, b_seg;
    const int32_t* order;
    int lda, ldb, m0, n0, last_m, last_n, w, wm, wn, lane;

    __device__ void seek_a(int seg) {
        const int kind = seg % kinds, k = seg / kinds;
        // wave-uniform (the buffer resource built from it must live in SGPRs)
        const int s = order ? __builtin_amdgcn_readfirstlane(order[k]) : k;
        abase = kind ? a_base1 : a_base0;
        a = abase + (int64_t)s * a_seg;
    }
    const uint16_t* abase = nullptr;                    // the current segment kind's A base
    __device__ void seek_b(int seg) {
        const int kind = seg % kinds, k = seg / kinds;
        b = (kind ? b_base1 : b_base0) + (int64_t)k * b_seg;
    }
    __device__ void issue_a(int g, uint16_t* lds_stage) {
        const int blk = g * NW + w;
        if constexpr (FRAG) {
            // block blk of the stage: 32-row block m0 / 32 + blk / 2, the
            // stage's 16-index block blk % 2 (m0 % 256 == 0, M % 256 == 0)
            const int64_t off = (int64_t)(m0 / 32 + (blk >> 1)) * 32 * lda + (int64_t)(a - abase) * 32 +
                                (blk & 1) * 512 + lane * 8;
            TSP_LDS void* dst = (TSP_LDS void*)(lds_stage + blk * 512);
            if constexpr (BUF) {
                const __amdgpu_buffer_rsrc_t rs =
                    __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, 0x7fffffff, kRawBufferWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (int)(off * 2), 0, 0, 0);
            } else {
                __builtin_amdgcn_global_load_lds(abase + off, dst, 16, 0, 0);
            }
        } else {
            load_rows<BUF>(lds_stage + blk * 512, a, lda, m0 + blk * 16, last_m, lane);
        }
    }
    __device__ void advance_a() {
        if (ls + 1 < spp) {
            ++ls;
            a += 32;
        } else if (j + 1 < nseg) {
            ls = 0;
            seek_a(++j);
        }
    }
    __device__ void issue_b(int g, uint16_t* lds_super, int h) {
        const int r0 = h * (BN / 2) + (g * NW + w) * 8;
        load_rows128<BUF>(lds_super + r0 * 64, b, ldb, n0 + r0, last_n, lane);
    }
    __device__ void advance_b() {
        if (lsb + 2 < spp) {
            lsb += 2;
            b += 64;
        } else if (jb + 1 < nseg) {
            lsb = 0;
            seek_b(++jb);
        }
    }
    __device__ void read_a(int q, const uint16_t* lds_stage, bf16x8 (&af)[TM]) const {
        if constexpr (FRAG) {
            // as PackedSrc::read_a: 16-row block ib = rows 16 (ib % 2) + l % 16
            // of 32-row block ib / 2, indices 8 (l / 16) .. + 7
            const int r = lane & 15, c = lane >> 4;
            const bf16x8* as = reinterpret_cast<const bf16x8*>(lds_stage);
            const int ib = wm * TM + q;
            af[q] = as[((ib >> 1) * 2 + (c >> 1)) * 64 + (c & 1) * 32 + (ib & 1) * 16 + r];
        } else {
            af[q] = read_rows(lds_stage, wm * TM + q, lane);
        }
    }
};

// A 256 x 256 tile's accumulators in the saved-activation layout: wave w's
// accumulator (i, j) of lane l is the f32x4 at ((tile * NW + w) * 64 +
// i * TN + j) * 64 + l, so that each store or load instruction moves 1 KiB of
// contiguous memory. Each instruction's base is wave-uniform (scalar
// registers) and the lane offset the only vector address, which keeps the
// 64 stores from tying up vector registers for addresses. Nontemporal both
// ways: a forward writes them for a backward that runs much later.
__device__ __forceinline__ void save_acc(float* __restrict__ base, int64_t tile, int w, int lane,
                                         const f32x4 (&acc)[TM][TN]) {
    f32x4* p = reinterpret_cast<f32x4*>(base) + (tile * NW + w) * (TM * TN * 64);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            f32x4* q = static_cast<f32x4*>(uniform_ptr(p + (i * TN + j) * 64));
            __builtin_nontemporal_store(acc[i][j], q + lane);
        }
}
__device__ __forceinline__ void load_acc(const float* __restrict__ base, int64_t tile, int w, int lane,
                                         f32x4 (&acc)[TM][TN]) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + (tile * NW + w) * (TM * TN * 64);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const f32x4* q = static_cast<const f32x4*>(uniform_ptr(p + (i * TN + j) * 64));
            acc[i][j] = __builtin_nontemporal_load(q + lane);
        }
}

// Ring bookkeeping: byte-free element offsets of the stage/super-stage that
// step t loads into and the one whose fragments it reads.
struct Ring {
    int a_ld = 0, a_rd = A_STAGE;                       // A buffers: loads of stage t + 4, reads of t + 1
    int b_ld = 2 * B_SUPER, b_rd = 0;                   // B buffers: loads of half t + 5, reads of t + 1
};
__device__ __forceinline__ int next_a(int off) { return off == (NA - 1) * A_STAGE ? 0 : off + A_STAGE; }
__device__ __forceinline__ int next_b(int off) { return off == (NB - 1) * B_SUPER ? 0 : off + B_SUPER; }

// Step t, H = (t + 1) % 2. The barrier makes every wave's share of step t + 1's
// data visible and ends every wave's fragment reads of step t (issued in step
// t - 1). The wave then loads A stage t + 4 into the A buffer step t read and
// half H of B super-stage (t + 5) / 2 (half t + 5 of the B stream) into the B
// buffer that super-stage (t + 5) / 2 - 3 held, whose last step (t - 1 or t)
// has been read; it reads step t + 1's fragments into the other register set
// while its MFMAs run on step t's, and before the next barrier waits for those
// reads and for every load it issued up to step t - 1 (step t + 2's data: A
// stage t + 2 was issued in step t - 2, the two halves of its B super-stage in
// steps t - 4 .. t - 2). Every step issues its loads (past the end, the last
// stage again, into a buffer nobody reads), so that wait is always "at most
// two steps' loads outstanding". FIRST: the accumulators start from 0. LAST:
// MFMAs only.
//
// With one wave per SIMD nothing else feeds the matrix pipe while this wave
// issues other work, so scheduling fences fix the order: three MFMAs right
// after the barrier, then eight groups of one load, two fragment reads and
// seven MFMAs (a load right after another costs the matrix pipe far more
// than one that follows a few MFMAs), and the scalar bookkeeping for the next
// step spread over the last five MFMAs.
template <bool FIRST, bool LAST, int H, class Src>
__device__ __forceinline__ void step(Ring& rg, Src& src, uint16_t* lds, f32x4 (&acc)[TM][TN],
                                     const bf16x8 (&ca)[TM], const bf16x8 (&cb)[TN], bf16x8 (&na)[TM],
                                     bf16x8 (&nb)[TN]) {
    constexpr int LEAD = 3, GROUP = 7;
    constexpr int TAIL = TM * TN - LEAD - LOADS * GROUP;
    static_assert(TM + TN == 2 * LOADS && TAIL == 5, "schedule");
    auto mf = [&](int m) {
        const int i = m / TN, j = (i & 1) ? TN - 1 - m % TN : m % TN;   // snake order
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[i], cb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f}
                                                                                : acc[i][j], 0, 0, 0);
    };
    if constexpr (LAST) {
#pragma unroll
        for (int m = 0; m < TM * TN; ++m) mf(m);
        // the epilogue starts after every MFMA: MFMAs sunk into it keep the
        // fragment registers alive there and made the compiler spill
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    const int a_ld = rg.a_ld, a_rd = rg.a_rd, b_ld = rg.b_ld, b_rd = rg.b_rd;
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < LEAD; ++m) mf(m);
    __builtin_amdgcn_sched_barrier(0);
    const int lane = src.lane;
#pragma unroll
    for (int g = 0; g < LOADS; ++g) {
        const int m0 = LEAD + GROUP * g;
        if (g < LA) src.issue_a(g, lds + a_ld);
        else src.issue_b(g - LA, lds + B_OFF + b_ld, H);
        mf(m0);
        mf(m0 + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (g < TM / 2) src.read_a(2 * g, lds + a_rd, na);
        else nb[2 * g - TM] = read_rows128(lds + B_OFF + b_rd, src.wn * TN + 2 * g - TM, H, lane);
        mf(m0 + 2);
        mf(m0 + 3);
        __builtin_amdgcn_sched_barrier(0);
        if (g < TM / 2) src.read_a(2 * g + 1, lds + a_rd, na);
        else nb[2 * g + 1 - TM] = read_rows128(lds + B_OFF + b_rd, src.wn * TN + 2 * g + 1 - TM, H, lane);
        mf(m0 + 4);
        mf(m0 + 5);
        mf(m0 + 6);
        __builtin_amdgcn_sched_barrier(0);
    }
    src.advance_a();
    rg.a_ld = a_rd;
    rg.a_rd = next_a(a_rd);
    if constexpr (H == 1) {                             // the next loads go to a new super-stage
        src.advance_b();
        rg.b_ld = next_b(b_ld);
    }
    if constexpr (H == 1) rg.b_rd = next_b(b_rd);       // the next step reads a new super-stage
#pragma unroll
    for (int m = TM * TN - TAIL; m < TM * TN; ++m) mf(m);
#pragma unroll
    for (int k = 0; k < TAIL; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x006, 4, 0);   // VALU / SALU
    }
    __builtin_amdgcn_sched_barrier(0);
    TSP_VMCNT(2 * LOADS);                               // own loads up to step t - 1 landed
    lgkm_zero();                                        // step t + 1's fragments in registers
    __builtin_amdgcn_sched_barrier(0);
}

// The reduction over ksteps steps (even, >= 2) of 32 indices on the split
// ring. src is positioned at step 0 for both operands. The prologue issues B
// half 0, then (A stage s, B half s + 1) for s = 0..3, exactly as steps
// -5..-1 would, and reads step 0's fragments. (Issuing a whole B super-stage
// every other step instead, which gives it 3 steps to land, measured slower
// for both products.)
template <class Src>
__device__ __forceinline__ void mainloop(uint16_t* lds, f32x4 (&acc)[TM][TN], int ksteps, Src& src) {
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    const int lane = src.lane;
#pragma unroll
    for (int g = 0; g < LB; ++g) src.issue_b(g, lds + B_OFF, 0);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
        const int u = s + 1;                            // B half u: super-stage u / 2, half u % 2
#pragma unroll
        for (int g = 0; g < LA; ++g) src.issue_a(g, lds + s * A_STAGE);
        src.advance_a();
#pragma unroll
        for (int g = 0; g < LB; ++g) src.issue_b(g, lds + B_OFF + (u >> 1) * B_SUPER, u & 1);
        if (u & 1) src.advance_b();
    }
    TSP_VMCNT(3 * LOADS);                               // A stage 0 and B super-stage 0 landed
    stage_barrier();
#pragma unroll
    for (int q = 0; q < TM; ++q) src.read_a(q, lds, a0);
#pragma unroll
    for (int q = 0; q < TN; ++q) b0[q] = read_rows128(lds + B_OFF, src.wn * TN + q, 0, lane);
    TSP_VMCNT(2 * LOADS + LB);                          // A stage 1 landed too
    lgkm_zero();
    __builtin_amdgcn_sched_barrier(0);

    Ring rg;
    step<true, false, 1>(rg, src, lds, acc, a0, b0, a1, b1);
    for (int t = 1; t + 2 < ksteps; t += 2) {
        step<false, false, 0>(rg, src, lds, acc, a1, b1, a0, b0);
        step<false, false, 1>(rg, src, lds, acc, a0, b0, a1, b1);
    }
    step<false, true, 0>(rg, src, lds, acc, a1, b1, a0, b0);
    TSP_VMCNT(0);                                       // no load into LDS outlives the workgroup
    __builtin_amdgcn_sched_barrier(0);
}

// ---- the 5-stage ring -------------------------------------------------------
// Both operands in 32-deep stages of 32 KiB ([A 16 KiB][B 16 KiB], B as
// sixteen 16-row x 64-byte blocks), five stages in the 160 KiB: step t loads
// stage t + 5 into the buffer stage t held, and before the next barrier waits
// only for stage t + 2, issued in step t - 3, so a load has three steps to land
// (two in the split ring). The price is the B loads' 64-byte row pieces: 16
// cache-line requests per instruction instead of 8. The down product, whose
// operands (H and the down weights) stream from beyond the L2, runs faster on
// this ring; the gate/up product on the split one (measured on one box).
constexpr int R5_STAGE = 2 * A_STAGE;
constexpr int NS5 = 5;
static_assert(NS5 * R5_STAGE <= LDS_ELEMS, "LDS");

__device__ __forceinline__ int next5(int off) { return off == (NS5 - 1) * R5_STAGE ? 0 : off + R5_STAGE; }

template <bool FIRST, bool LAST, class Src>
__device__ __forceinline__ void step5(int& ld_ref, int& rd_ref, Src& src, uint16_t* lds, f32x4 (&acc)[TM][TN],
                                      const bf16x8 (&ca)[TM], const bf16x8 (&cb)[TN], bf16x8 (&na)[TM],
                                      bf16x8 (&nb)[TN]) {
    constexpr int LEAD = 3, GROUP = 7;
    constexpr int TAIL = TM * TN - LEAD - LOADS * GROUP;
    auto mf = [&](int m) {
        const int i = m / TN, j = (i & 1) ? TN - 1 - m % TN : m % TN;   // snake order
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
    const int lane = src.lane;
#pragma unroll
    for (int g = 0; g < LOADS; ++g) {
        const int m0 = LEAD + GROUP * g;
        if (g < LA) src.issue_a(g, lds + ld_off);
        else src.issue_b32(g - LA, lds + ld_off + A_STAGE);
        mf(m0);
        mf(m0 + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (g < TM / 2) src.read_a(2 * g, lds + rd_off, na);
        else nb[2 * g - TM] = read_rows(lds + rd_off + A_STAGE, src.wn * TN + 2 * g - TM, lane);
        mf(m0 + 2);
        mf(m0 + 3);
        __builtin_amdgcn_sched_barrier(0);
        if (g < TM / 2) src.read_a(2 * g + 1, lds + rd_off, na);
        else nb[2 * g + 1 - TM] = read_rows(lds + rd_off + A_STAGE, src.wn * TN + 2 * g + 1 - TM, lane);
        mf(m0 + 4);
        mf(m0 + 5);
        mf(m0 + 6);
        __builtin_amdgcn_sched_barrier(0);
    }
    src.advance5();
    ld_ref = rd_off;
    rd_ref = next5(rd_off);
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

// The reduction over ksteps stages (even, >= 2) on the 5-stage ring; src is
// positioned at stage 0 for both operands (issue_a / issue_b32).
template <class Src>
__device__ __forceinline__ void mainloop5(uint16_t* lds, f32x4 (&acc)[TM][TN], int ksteps, Src& src) {
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    const int lane = src.lane;
#pragma unroll
    for (int t = 0; t < NS5; ++t) {
#pragma unroll
        for (int g = 0; g < LA; ++g) src.issue_a(g, lds + t * R5_STAGE);
#pragma unroll
        for (int g = 0; g < LOADS - LA; ++g) src.issue_b32(g, lds + t * R5_STAGE + A_STAGE);
        src.advance5();
    }
    TSP_VMCNT((NS5 - 1) * LOADS);                       // own loads of stage 0 landed
    stage_barrier();
#pragma unroll
    for (int q = 0; q < TM; ++q) src.read_a(q, lds, a0);
#pragma unroll
    for (int q = 0; q < TN; ++q) b0[q] = read_rows(lds + A_STAGE, src.wn * TN + q, lane);
    TSP_VMCNT((NS5 - 2) * LOADS);                       // own loads of stage 1 landed
    lgkm_zero();
    __builtin_amdgcn_sched_barrier(0);
    int ld = 0, rd = R5_STAGE;                          // buffers of stages t and t + 1
    step5<true, false>(ld, rd, src, lds, acc, a0, b0, a1, b1);
    for (int t = 1; t + 2 < ksteps; t += 2) {
        step5<false, false>(ld, rd, src, lds, acc, a1, b1, a0, b0);
        step5<false, false>(ld, rd, src, lds, acc, a0, b0, a1, b1);
    }
    step5<false, true>(ld, rd, src, lds, acc, a1, b1, a0, b0);
    TSP_VMCNT(0);                                       // no load into LDS outlives the workgroup
}

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
    static_assert(ELEMS * 2 <= LDS_ELEMS * 2, "LDS");
    uint16_t* lds;
    __device__ __forceinline__ void put4(int r, int c, uint2 v) {
        *reinterpret_cast<uint2*>(lds + r * PITCH + c) = v;
    }
    // The staged 256-row tile into H's 16-token x 32-column blocks (see
    // Bf16Args::nbt): one whole 1 KiB block per store instruction; the tile's
    // columns start at column block kb0; token blocks past nbt are skipped.
    __device__ __forceinline__ void flush_blocks(uint16_t* __restrict__ dst, int nbt, int t0, int64_t kb0, int w,
                                                 int lane) const {
        static_assert(ROWS == 256 && COLS % 32 == 0, "blocked flush");
        constexpr int NCB = COLS / 32, NBLK = (ROWS / 16) * NCB;
        const int r = lane >> 2, c = lane & 3;
#pragma unroll 4
        for (int it = 0; it < NBLK / 4; ++it) {
            const int blk = it * 4 + w;
            const int i = blk % (ROWS / 16), j = blk / (ROWS / 16);   // token block, column block
            const int tb = (t0 >> 4) + i;
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (i * 16 + r) * PITCH + j * 32 + c * 8);
            if (tb < nbt) *reinterpret_cast<u32x4*>(dst + ((kb0 + j) * nbt + tb) * 512 + lane * 8) = v;
        }
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

// Half hh of a StagedRows16<COLS, 128> tile, transposed, into dst (COLS rows
// of ldt tokens, tokens contiguous) at rows row0 + c and the half's token
// columns: staged row r is tile row (r / 64) * 128 + hh * 64 + r % 64. Four
// lanes take one column, each 8 consecutive tokens (8 LDS reads of 2 bytes),
// and store them as 16 bytes, so that a store instruction writes 64
// contiguous bytes of each of 16 rows; columns t0 + tile row >= ldt are
// skipped. A read instruction touches 16 neighbouring columns of 4 rows 8
// apart, whose words fall on two bank sets (8 rows are a multiple of 32 banks
// away); the lanes of rows 16 apart take columns 16 further on, so that the
// four rows' reads use four bank sets (23 % of the LDS cycles were conflicts).
template <int COLS>
__device__ __forceinline__ void flush_transposed(const StagedRows16<COLS, 128>& stg, uint16_t* __restrict__ dst,
                                                 int64_t ldt, int64_t row0, int t0, int hh, int tid) {
    constexpr int PITCH = StagedRows16<COLS, 128>::PITCH;
    // a 4-lane group covers 32 tokens of one column; 4 such token quarters
    // per staged half, 16 columns per wave per pass
#pragma unroll 2
    for (int it = 0; it < COLS / 16; ++it) {
        const int id = it * 256 + tid;
        const int q = id & 3, tq = id / (4 * COLS);    // tq: which 32 tokens
        const int c = (((id >> 2) & (COLS - 1)) + 16 * (q >> 1)) & (COLS - 1);
        const int r = tq * 32 + q * 8;                      // first staged row of the lane's 8 tokens
        const int col = t0 + (r >> 6) * 128 + hh * 64 + (r & 63);
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)stg.lds[(r + 2 * e) * PITCH + c] | ((uint32_t)stg.lds[(r + 2 * e + 1) * PITCH + c] << 16);
        if (col < ldt) *reinterpret_cast<u32x4*>(dst + (row0 + c) * ldt + col) = u32x4{v[0], v[1], v[2], v[3]};
    }
}

// Half hh of a StagedRows16<COLS, 128> tile, transposed, into dst stored in
// 32 x 16 fragment blocks (rows = the tile's columns at row0 + c, reduction
// index = token, KB = ldt / 16 blocks per 32-row block; see RowSrc<.., FRAG>):
// a lane takes one column and 8 consecutive tokens, i.e. one 16-byte lane slot
// of a block. The 64 lanes of a wave take 64 neighbouring columns of the same
// 8 staged rows (LDS reads of one 128-byte row segment: no bank conflicts) and
// store two runs of 512 contiguous bytes; tokens >= ldt are skipped.
template <int COLS>
__device__ __forceinline__ void flush_frag_transposed(const StagedRows16<COLS, 128>& stg, uint16_t* __restrict__ dst,
                                                      int64_t ldt, int64_t row0, int t0, int hh, int tid) {
    constexpr int PITCH = StagedRows16<COLS, 128>::PITCH;
    static_assert(COLS % 64 == 0, "frag flush");
    const int64_t kb_per_row = ldt >> 4;
#pragma unroll 2
    for (int it = 0; it < COLS / 16; ++it) {
        const int id = it * 256 + tid;
        const int c = id % COLS, r = (id / COLS) * 8;           // column, first staged row of the 8 tokens
        const int col = t0 + (r >> 6) * 128 + hh * 64 + (r & 63);
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)stg.lds[(r + 2 * e) * PITCH + c] | ((uint32_t)stg.lds[(r + 2 * e + 1) * PITCH + c] << 16);
        const int64_t row = row0 + c;
        const int64_t off = ((row >> 5) * kb_per_row + (col >> 4)) * 512 + ((row & 31) + 32 * ((col >> 3) & 1)) * 8;
        if (col < ldt) *reinterpret_cast<u32x4*>(dst + off) = u32x4{v[0], v[1], v[2], v[3]};
    }
}

// The fp32 counterpart for 256-column result tiles: 128 staged rows, one half
// hh of each wave row's tokens (as StagedRows16<COLS, 128>), 1 KiB per row so
// that each flush store writes one whole row. put4 takes one lane's four
// values; the pitch 260 puts a put4 instruction's 16 rows 4 banks apart.
struct StagedRowsF32 {
    static constexpr int COLS = 256, ROWS = 128, PITCH = COLS + 4;
    static constexpr int ELEMS = ROWS * PITCH;          // floats
    static_assert(ELEMS * 4 <= LDS_ELEMS * 2, "LDS");
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

#undef TSP_VMCNT

}  // namespace w16
}  // namespace tsp
