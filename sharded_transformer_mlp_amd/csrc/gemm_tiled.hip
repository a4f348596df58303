// Tiled bf16 MFMA kernels of the sharded MLP (gfx950).
//
// Both products run with the weights as the MFMA A operand (rows = output
// features) and the tokens as the B operand (columns = tokens), using
// v_mfma_f32_32x32x16_bf16. Each lane then holds, per 32 x 32 block, four
// runs of 4 consecutive output features of one token, so the epilogue writes
// H (bf16) and Y (fp32) rows straight from registers.
//
// gateup_tiled: H_k = act(X . W_{order[k]}) for every ring step k, the
//   SwiGLU or GeLU epilogue applied in registers ("Tensor Parallelism:
//   Splitting the Math", section "Why the column-then-row split": the
//   nonlinearity is exact on a shard's own columns). Packed records and the
//   hidden columns of the workspace are both in ring order, so H_k occupies
//   columns [k*F, (k+1)*F). Tiles of ring step k are dispatched before those
//   of step k + 1.
// down_tiled:   Y = sum_k H_k . Wd_{order[k]}; the reduction loop walks the
//   records in ring order and keeps the fp32 Y tile in registers for the
//   whole walk, so Y is written once ("Folding Tensor and Sequence
//   Parallelism ...", Abstract: partial outputs accumulate locally).
//
// Shapes 1-3 (smaller tiles, for token counts and shard widths that 256 x 256
// tiles would leave with too few workgroups): 32 reduction indices per
// stage, global memory loaded into registers two stages ahead and written to
// a 3-deep LDS ring laid out in fragment blocks, so every operand fragment
// read is one contiguous (or XOR-swizzled) 16-byte-per-lane access without
// bank conflicts; the waves run a two-group ping-pong (see mainloop): on every
// SIMD one wave issues MFMAs while the other moves data. Shape 0 (w16.h, the
// automatic choice at large T) loads global memory straight into LDS, uses
// 16x16x32 MFMAs and runs one wave per SIMD holding a 128 x 128 piece in all
// 256 accumulation registers; it measured fastest on every large-T workload.
#include "common.h"
#include "launch.h"
#include "w16.h"

namespace tsp {


template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN;                   // waves
    static constexpr int NT = NW * 64;                   // threads
    static constexpr int TM = BM / WM / 32;              // 32-row MFMA blocks per wave (features)
    static constexpr int TN = BN / WN / 32;              // 32-column MFMA blocks per wave (tokens)
    static constexpr int A_BLK = BM / 16;                // 1 KiB blocks per stage (A)
    static constexpr int B_BLK = BN / 16;                // (B)
    static constexpr int LA = A_BLK / NW;                // A blocks each wave loads per stage
    static constexpr int LB = B_BLK / NW;                // B blocks each wave loads per stage
    static constexpr int STAGE = (A_BLK + B_BLK) * 512;  // bf16 elements per stage (32-deep)
    static constexpr int NS = 3;                         // stages in the LDS ring
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(LA * NW == A_BLK && LB * NW == B_BLK, "loader split");
    static_assert(NS * STAGE * 2 <= 160 * 1024, "LDS");
};


// LDS layout of one stage (32 reduction indices):
//   A blocks are the packed 32 x 16 fragment blocks, already in MFMA order:
//   stage block b < A_BLK is (row block b / 2, reduction block b % 2).
//   B blocks hold 16 tokens x the stage's 32 reduction indices, so one wave
//   load reads 16 whole 64-byte row pieces of X (or H). Inside a block, token
//   r's 8-index chunk c sits in 16-byte slot 4 r + (c ^ ((r >> 2) & 3)); the
//   XOR keeps both the writes and the MFMA fragment reads (16 tokens x one
//   chunk per lane group) free of LDS bank conflicts.
__device__ __forceinline__ int tok_slot(int r, int c) { return 4 * r + (c ^ ((r >> 2) & 3)); }

// One stage's share of global data for one thread: up to two A and two B
// 16-byte pieces, as named members (register arrays of two elements are not
// reliably kept in registers by the compiler).
struct StageRegs {
    u32x4 a0, a1, b0, b1;
};

// Global loads of one stage into registers. Each wave loads whole 1 KiB
// blocks (block i * NW + w). Token rows past T are clamped to row T - 1
// (their outputs are never stored).
template <class C>
__device__ __forceinline__ void load_stage(StageRegs& r, const uint16_t* __restrict__ a_base, int64_t a_rs,
                                           const uint16_t* __restrict__ b_src, int ldb, int64_t b_koff,
                                           int t0, int T, int w, int lane) {
    static_assert(C::LA >= 1 && C::LA <= 2 && C::LB >= 1 && C::LB <= 2, "stage split");
    auto a_ptr = [&](int i) {
        const int b = i * C::NW + w;
        return reinterpret_cast<const u32x4*>(a_base + (b >> 1) * a_rs + (b & 1) * 512 + lane * 8);
    };
    auto b_ptr = [&](int i) {
        const int bb = i * C::NW + w;
        const int tok = min(t0 + bb * 16 + (lane >> 2), T - 1);
        return reinterpret_cast<const u32x4*>(b_src + (int64_t)tok * ldb + b_koff + (lane & 3) * 8);
    };
    r.a0 = *a_ptr(0);
    if constexpr (C::LA > 1) r.a1 = *a_ptr(1);
    r.b0 = *b_ptr(0);
    if constexpr (C::LB > 1) r.b1 = *b_ptr(1);
}

template <class C>
__device__ __forceinline__ void store_stage(uint16_t* lds_stage, const StageRegs& r, int w, int lane) {
    u32x4* as = reinterpret_cast<u32x4*>(lds_stage);
    u32x4* bs = reinterpret_cast<u32x4*>(lds_stage + C::A_BLK * 512);
    const int slot = tok_slot(lane >> 2, lane & 3);
    as[w * 64 + lane] = r.a0;
    if constexpr (C::LA > 1) as[(C::NW + w) * 64 + lane] = r.a1;
    bs[w * 64 + slot] = r.b0;
    if constexpr (C::LB > 1) bs[(C::NW + w) * 64 + slot] = r.b1;
}

__device__ __forceinline__ void vmcnt_le(int n) {
    // s_waitcnt with vmcnt = n (n <= 15), expcnt / lgkmcnt left at their maximum
    if (n >= 8) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
    else if (n >= 3) __builtin_amdgcn_s_waitcnt(3 | (7 << 4) | (15 << 8));
    else if (n >= 2) __builtin_amdgcn_s_waitcnt(2 | (7 << 4) | (15 << 8));
    else if (n >= 1) __builtin_amdgcn_s_waitcnt(1 | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}


template <class C>
__device__ __forceinline__ void read_frags(const uint16_t* lds_stage, bf16x8 (&af)[2][C::TM],
                                           bf16x8 (&bv)[2][C::TN], int wm, int wn, int lane) {
    const bf16x8* as = reinterpret_cast<const bf16x8*>(lds_stage);
    const bf16x8* bs = reinterpret_cast<const bf16x8*>(lds_stage + C::A_BLK * 512);
    // B fragment (32 tokens x 16 indices): lane l takes token l % 32, i.e.
    // block 2 j' + (l / 16) % 2, row l % 16, chunk 2 kk + l / 32.
    const int r = lane & 15, half = (lane >> 4) & 1, hi = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) af[kk][i] = as[((wm * C::TM + i) * 2 + kk) * 64 + lane];
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            bv[kk][j] = bs[((wn * C::TN + j) * 2 + half) * 64 + tok_slot(r, 2 * kk + hi)];
    }
}

template <class C>
__device__ __forceinline__ void mfma_stage(f32x16 (&acc)[C::TM][C::TN], const bf16x8 (&af)[2][C::TM],
                                           const bf16x8 (&bv)[2][C::TN]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
}

// The reduction loop shared by both kernels. `src(t, a_base, b_koff)` gives
// step t's A slab start and B reduction offset (32 indices per step).
//
// Ping-pong schedule: the waves form two groups (waves 0..NW/2-1 and the
// rest), one wave of each group per SIMD. Step t is a memory phase M(t) and
// a compute phase C(t) (the MFMAs). Group 1 runs one phase behind group 0,
// and every phase boundary is a workgroup barrier, so on each SIMD one wave
// computes while the other does its memory work. Barrier b_{2t} opens group
// 0's M(t); b_{2t+1} opens group 0's C(t) and group 1's M(t).
//
// M(t): wait for the registers holding stage t + 2 (loaded in M(t-2)), write
// them to LDS buffer (t + 2) % 3, load stage t + 4 into them, read stage t's
// fragments, and drain the LDS traffic (lgkmcnt 0) before the next barrier.
// Exactly one stage of loads is issued per step, so "stage t + 2 landed" is
// always vmcnt <= loads-per-stage.
// Stage t + 2's buffer was last read by M(t-1) of both groups, which ended
// before b_{2t}; stage t was written in M(t-2) of both groups, which ended
// before b_{2t-1}. Two register sets hold the stages in flight, so the loop
// is unrolled by two.
// One step of the ping-pong loop for the register set rr that holds stage
// t + 2 (see mainloop).
template <class C, class Src>
__device__ __forceinline__ void pp_step(int t, int K, uint16_t* lds, StageRegs& rr,
                                        f32x16 (&acc)[C::TM][C::TN], int64_t a_rs, const uint16_t* b_src,
                                        int ldb, int t0, int T, int w, int wm, int wn, int lane, Src& src) {
    constexpr int LPS = C::LA + C::LB;                  // global loads per stage per thread
    bf16x8 af[2][C::TM], bv[2][C::TN];
    stage_barrier();                                    // g0: b_{2t}, g1: b_{2t+1}
    __builtin_amdgcn_sched_barrier(0);
    // Unconditional: past the end the loads fetch the last stage again and
    // the stores fill a free buffer that is never read, so the compiler sees
    // one fixed load order and keeps the two stages in flight.
    vmcnt_le(LPS);                                      // stage t + 2 landed in rr
    store_stage<C>(lds + ((t + 2) % C::NS) * C::STAGE, rr, w, lane);
    {
        const uint16_t* ab;
        int64_t bk;
        src(min(t + 4, K - 1), ab, bk);
        load_stage<C>(rr, ab, a_rs, b_src, ldb, bk, t0, T, w, lane);
    }
    read_frags<C>(lds + (t % C::NS) * C::STAGE, af, bv, wm, wn, lane);
    lgkm_zero();
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();                                    // g0: b_{2t+1}, g1: b_{2t+2}
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    mfma_stage<C>(acc, af, bv);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
}

// The reduction loop shared by both kernels. `src(t, a_base, b_koff)` gives
// step t's A slab start and B reduction offset (32 indices per step).
//
// Ping-pong schedule: the waves form two groups (waves 0..NW/2-1 and the
// rest), one wave of each group per SIMD. Step t is a memory phase M(t) and
// a compute phase C(t) (the MFMAs). Group 1 runs one phase behind group 0,
// and every phase boundary is a workgroup barrier, so on each SIMD one wave
// computes while the other does its memory work. Barrier b_{2t} opens group
// 0's M(t); b_{2t+1} opens group 0's C(t) and group 1's M(t).
//
// M(t): wait for the registers holding stage t + 2 (loaded in M(t-2)), write
// them to LDS buffer (t + 2) % 3, load stage t + 4 into them, read stage t's
// fragments, and drain the LDS traffic (lgkmcnt 0) before the next barrier.
// Exactly one stage of loads is issued per step, so "stage t + 2 landed" is
// always vmcnt <= loads-per-stage.
// Stage t + 2's buffer was last read by M(t-1) of both groups, which ended
// before b_{2t}; stage t was written in M(t-2) of both groups, which ended
// before b_{2t-1}. Two register sets hold the stages in flight, so the loop
// is unrolled by two.
template <class C, class Src>
__device__ __forceinline__ void mainloop(uint16_t* lds, f32x16 (&acc)[C::TM][C::TN], int K,
                                         int64_t a_rs, const uint16_t* b_src, int ldb, int t0, int T,
                                         Src src) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = w / C::WN, wn = w % C::WN;
    const bool g1 = w >= C::NW / 2;
    constexpr int LPS = C::LA + C::LB;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    StageRegs r0, r1;
    const uint16_t* ab;
    int64_t bk;
    // prologue: stages 0 and 1 go to LDS, stages 2 and 3 stay in registers
    // (stage indices past the end are clamped; that data is never read)
    src(0, ab, bk);
    load_stage<C>(r0, ab, a_rs, b_src, ldb, bk, t0, T, w, lane);
    src(min(1, K - 1), ab, bk);
    load_stage<C>(r1, ab, a_rs, b_src, ldb, bk, t0, T, w, lane);
    vmcnt_le(LPS);
    store_stage<C>(lds, r0, w, lane);
    vmcnt_le(0);
    store_stage<C>(lds + C::STAGE, r1, w, lane);
    // keep the issue order r0 then r1: the loop's waits count on it
    __builtin_amdgcn_sched_barrier(0);
    src(min(2, K - 1), ab, bk);
    load_stage<C>(r0, ab, a_rs, b_src, ldb, bk, t0, T, w, lane);
    __builtin_amdgcn_sched_barrier(0);
    src(min(3, K - 1), ab, bk);
    load_stage<C>(r1, ab, a_rs, b_src, ldb, bk, t0, T, w, lane);
    __builtin_amdgcn_sched_barrier(0);
    lgkm_zero();
    if (g1) stage_barrier();                            // b_0: group 1 sits out phase 0
    // K is even (d and F are multiples of 64): both unrolled steps always
    // run, so no path through the loop skips a load, and the compiler's
    // wait analysis sees the same load order on every edge.
    for (int t = 0; t < K; t += 2) {
        pp_step<C>(t, K, lds, r0, acc, a_rs, b_src, ldb, t0, T, w, wm, wn, lane, src);
        pp_step<C>(t + 1, K, lds, r1, acc, a_rs, b_src, ldb, t0, T, w, wm, wn, lane, src);
    }
    if (!g1) stage_barrier();                           // b_{2K}: group 0 matches group 1's count
}

template <class C, class Src>
__device__ __forceinline__ void run_mainloop(uint16_t* lds, f32x16 (&acc)[C::TM][C::TN], int K,
                                             int64_t a_rs, const uint16_t* b_src, int ldb, int t0, int T,
                                             Src src) {
    mainloop<C>(lds, acc, K, a_rs, b_src, ldb, t0, T, src);
}

// act: 1 = SwiGLU (packed 32-row blocks alternate gate / up), 2 = GeLU (tanh form)
template <int BM, int BN, int WM, int WN, int ACT>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void gateup_tiled(Bf16Args a, int n_ft_shard, int n_tt) {
    using C = TileCfg<BM, BN, WM, WN>;
    static_assert(ACT != 1 || C::TM % 2 == 0, "SwiGLU pairs gate and up blocks inside a wave");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];
    poison_lds(lds, sizeof(lds));

    int ttile, flin;
    raster(xcd_remap(blockIdx.x, gridDim.x), a.P * n_ft_shard, n_tt, ttile, flin);
    const int s = flin / n_ft_shard;                    // ring step = packed record
    const int ftile = flin - s * n_ft_shard;
    const int64_t a_rs = (int64_t)(a.d >> 4) * 512;     // elements per 32-row block row
    const uint16_t* a_tile = a.packed + (int64_t)s * a.shard_elems + (int64_t)(ftile * (BM / 32)) * a_rs;
    const int t0 = ttile * BN;

    f32x16 acc[C::TM][C::TN];
    run_mainloop<C>(lds, acc, a.d >> 5, a_rs, a.x, a.d, t0, a.T,
                [&](int t, const uint16_t*& ab, int64_t& bk) {
                    ab = a_tile + (int64_t)t * 1024;
                    bk = (int64_t)t * 32;
                });

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    const int fsub = 4 * (lane >> 5);                   // feature offset inside each run of 8
    if constexpr (ACT == 1) {
#pragma unroll
        for (int p = 0; p < C::TM / 2; ++p) {
            const int gb = ftile * (BM / 32) + wm * C::TM + 2 * p;     // gate block (even)
            const int hbase = s * a.F + (gb >> 1) * 32 + fsub;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int tok = t0 + (wn * C::TN + j) * 32 + (lane & 31);
                if (tok < a.T) {
                    const f32x16 g = acc[2 * p][j], u = acc[2 * p + 1][j];
                    uint16_t* hrow = a.h + (int64_t)tok * a.f + hbase;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint2*>(hrow + 8 * q) =
                            pack4_bf16(silu_f(g[4 * q]) * u[4 * q], silu_f(g[4 * q + 1]) * u[4 * q + 1],
                                       silu_f(g[4 * q + 2]) * u[4 * q + 2], silu_f(g[4 * q + 3]) * u[4 * q + 3]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int hbase = s * a.F + (ftile * (BM / 32) + wm * C::TM + i) * 32 + fsub;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int tok = t0 + (wn * C::TN + j) * 32 + (lane & 31);
                if (tok < a.T) {
                    const f32x16 u = acc[i][j];
                    uint16_t* hrow = a.h + (int64_t)tok * a.f + hbase;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint2*>(hrow + 8 * q) =
                            pack4_bf16(gelu_tanh_f(u[4 * q]), gelu_tanh_f(u[4 * q + 1]),
                                       gelu_tanh_f(u[4 * q + 2]), gelu_tanh_f(u[4 * q + 3]));
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void down_tiled(Bf16Args a, int n_ft, int n_tt) {
    using C = TileCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];
    poison_lds(lds, sizeof(lds));

    int ttile, ftile;
    raster(xcd_remap(blockIdx.x, gridDim.x), n_ft, n_tt, ttile, ftile);
    const int spp = a.F >> 5;                           // 32-wide steps per shard
    const int64_t a_rs = (int64_t)(a.F >> 4) * 512;     // elements per 32-row block row
    const uint16_t* a_ft = a.packed + a.down_off + (int64_t)(ftile * (BM / 32)) * a_rs;
    const int t0 = ttile * BN;

    f32x16 acc[C::TM][C::TN];
    // Reduction step t is local step t % spp of ring step t / spp; records
    // and H columns are both stored in ring order, so this is a linear walk.
    run_mainloop<C>(lds, acc, a.P * spp, a_rs, a.h, a.f, t0, a.T,
                [&](int t, const uint16_t*& ab, int64_t& bk) {
                    const int k = t / spp, ls = t - k * spp;
                    ab = a_ft + (int64_t)k * a.shard_elems + (int64_t)ls * 1024;
                    bk = (int64_t)t * 32;
                });

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    const int fsub = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int n = ftile * BM + (wm * C::TM + i) * 32 + fsub;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int tok = t0 + (wn * C::TN + j) * 32 + (lane & 31);
            if (tok < a.T) {
                const f32x16 v = acc[i][j];
                float* yrow = a.y + (int64_t)tok * a.d + n;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4*>(yrow + 8 * q) =
                        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            }
        }
    }
}

// ------------------------------------------------------------------ shape 0
// The pipeline of w16.h with the forward's operands (PackedSrc): the gate/up
// product on the split ring (whole 128-byte token rows per load), the down
// product on the 5-stage ring (measured on one box, Llama shape: gate/up
// 683 -> 667 us and 70B long 11.56 -> 10.79 ms on the split ring; the down
// product 4-5 % slower there than on the 5-stage ring). Both measured faster
// than every variant of the ping-pong shapes, of staging operands through
// registers, and of a persistent grid that streams the next tile's first
// stages during the epilogue.

// SAVE: the accumulators (pre-activations) also go to a.save (w16::save_acc).
template <int ACT, bool BUF, bool BLK, bool SAVE>
__global__ __launch_bounds__(256) void gateup_w16(Bf16Args a, int n_ft_shard, int n_tt) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
    poison_lds(lds, sizeof(lds));
    int ttile, flin;
    raster(xcd_remap(blockIdx.x, gridDim.x), a.P * n_ft_shard, n_tt, ttile, flin, a.gt);
    const int s = flin / n_ft_shard;
    const int ftile = flin - s * n_ft_shard;
    const int64_t a_rs = (int64_t)(a.d >> 4) * 512;
    const uint16_t* a_tile = a.packed + (int64_t)s * a.shard_elems + (int64_t)(ftile * (BM / 32)) * a_rs;
    const int t0 = ttile * BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    PackedSrc<BUF> src{a_tile, 0, 0, a.d >> 5, 0, 0, a_rs, a.x, a.d, t0, a.T,
                       __builtin_amdgcn_readfirstlane(w), wm, wn, lane};
    f32x4 acc[TM][TN];
    w16::mainloop(lds, acc, a.d >> 5, src);

    // H through the LDS ring (StagedRows16): every wave's last fragment reads
    // are done at the first barrier, its LDS writes at the second
    const int fsub = 4 * (lane >> 4);
    stage_barrier();
    if constexpr (ACT == 1) {
        // the wave's 128 rows are two (32 gate, 32 up) row pairs: 16-row
        // blocks 4 q, 4 q + 1 gate and 4 q + 2, 4 q + 3 up of hidden group q;
        // the tile holds 128 hidden columns
        StagedRows16<BM / 2> stg{lds};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = (wm * 2 + q) * 32 + i * 16 + fsub;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const f32x4 g = acc[4 * q + i][j], u = acc[4 * q + 2 + i][j];
                    stg.put4((wn * TN + j) * 16 + (lane & 15), c,
                             pack4_bf16(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1], silu_f(g[2]) * u[2],
                                        silu_f(g[3]) * u[3]));
                }
            }
        lgkm_zero();
        stage_barrier();
        if constexpr (BLK) stg.flush_blocks(a.h, a.nbt, t0, ((int64_t)s * a.F + ftile * (BM / 2)) >> 5, w, lane);
        else stg.flush(a.h, a.f, t0, a.T, (int64_t)s * a.F + ftile * (BM / 2), w, lane);
    } else {
        StagedRows16<BM> stg{lds};
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int c = (wm * TM + i) * 16 + fsub;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const f32x4 u = acc[i][j];
                stg.put4((wn * TN + j) * 16 + (lane & 15), c,
                         pack4_bf16(gelu_tanh_f(u[0]), gelu_tanh_f(u[1]), gelu_tanh_f(u[2]), gelu_tanh_f(u[3])));
            }
        }
        lgkm_zero();
        stage_barrier();
        if constexpr (BLK) stg.flush_blocks(a.h, a.nbt, t0, ((int64_t)s * a.F + ftile * BM) >> 5, w, lane);
        else stg.flush(a.h, a.f, t0, a.T, (int64_t)s * a.F + ftile * BM, w, lane);
    }
    // the pre-activations for a backward, after the epilogue (the accumulators
    // are intact): the stores drain while the next tile starts on this CU
    // (measured: the training forward 1033 -> 1021 us against saving first)
    if constexpr (SAVE) save_acc(a.save, (int64_t)flin * n_tt + ttile, __builtin_amdgcn_readfirstlane(w), lane, acc);
}

template <bool BLK, bool BUF>
__global__ __launch_bounds__(256) void down_w16(Bf16Args a, int n_ft, int n_tt, int split) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
    poison_lds(lds, sizeof(lds));
    const int n_tiles = n_ft * n_tt;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int g = lin / n_tiles;
    int ttile, ftile;
    raster(lin - g * n_tiles, n_ft, n_tt, ttile, ftile, a.gt);
    const int spp = a.F >> 5;
    const int steps_per_group = a.P / split;
    const int64_t a_rs = (int64_t)(a.F >> 4) * 512;
    const uint16_t* a_ft = a.packed + a.down_off + (int64_t)(g * steps_per_group) * a.shard_elems +
                           (int64_t)(ftile * (BM / 32)) * a_rs;
    // the group's first hidden column: row-major, or its column block (BLK)
    const uint16_t* h_g = BLK ? a.h + (int64_t)(g * steps_per_group) * spp * a.nbt * 512
                              : a.h + (int64_t)(g * steps_per_group) * a.F;
    float* y = split > 1 ? a.part + (int64_t)g * a.T * a.d : a.y;
    const int t0 = ttile * BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    PackedSrc<BUF, BLK> src{a_ft, 0, 0, steps_per_group * spp, spp, a.shard_elems, a_rs, h_g, a.f, t0, a.T,
                              __builtin_amdgcn_readfirstlane(w), wm, wn, lane};
    src.set_blocked(a.nbt);
    f32x4 acc[TM][TN];
    w16::mainloop5(lds, acc, steps_per_group * spp, src);

    // Y rows through the LDS ring, half of each wave row's tokens at a time,
    // so that each store writes a whole 1 KiB row (from the MFMA layout a
    // store covers 16 tokens x 64 bytes)
    StagedRowsF32 stg{reinterpret_cast<float*>(lds)};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        stage_barrier();                                // fragment reads / the last flush's reads are done
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < TN / 2; ++jj)
                stg.put4(wn * 64 + jj * 16 + (lane & 15), (wm * TM + i) * 16 + 4 * (lane >> 4),
                         acc[i][hh * (TN / 2) + jj]);
        lgkm_zero();
        stage_barrier();
        stg.flush(y, a.d, t0, a.T, 0, (int64_t)ftile * BM, w, lane, hh);
        lgkm_zero();
    }
}

// Y = sum of the `split` partials, added in ring order (group 0 first).
__global__ __launch_bounds__(256) void reduce_partials(const float4* __restrict__ part, int split, int64_t n4,
                                                       float4* __restrict__ y) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        float4 s = part[i];
        for (int g = 1; g < split; ++g) {
            const float4 v = part[(int64_t)g * n4 + i];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        y[i] = s;
    }
}

// ------------------------------------------------------------------ configs
// cfg: 0 = 256 x 256, 16x16x32 MFMAs, 4 waves of 128 x 128 over global-to-LDS
//      loads (w16.h; the choice at large T), 1 = 256 x 128 (8 waves as 4 x 2,
//      32x32x16, register-staged ping-pong), 2 = 128 x 128 (4 waves as 2 x 2),
//      3 = 64 x 128 (4 waves as 1 x 4): the smaller tiles serve token counts
//      and shard widths that 256 x 256 tiles would leave with too few
//      workgroups, and shard widths that are not multiples of 256.
struct CfgDesc { int bm, bn; const char* name; };
constexpr int kNumCfgs = 4;
static const CfgDesc kCfgs[kNumCfgs] = {
    {256, 256, "256x256 16x16 4-wave"}, {256, 128, "256x128"}, {128, 128, "128x128"}, {64, 128, "64x128"}};

const char* tiled_cfg_name(int cfg) { return (cfg >= 0 && cfg < kNumCfgs) ? kCfgs[cfg].name : "none"; }

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool gateup_cfg_fits(int cfg, int d, int F, int swiglu) {
    if (cfg < 0 || cfg >= kNumCfgs) return false;
    const int64_t ngu = swiglu ? 2LL * F : (int64_t)F;
    return ngu % kCfgs[cfg].bm == 0 && d % 64 == 0;
}

bool down_cfg_fits(int cfg, int d, int F) {
    return cfg >= 0 && cfg < kNumCfgs && d % kCfgs[cfg].bm == 0 && F % 64 == 0;
}

// Automatic choice: the first shape in the list that divides the shard's
// packed width (gate/up) or d (down) and still gives at least one full wave
// of workgroups on 256 CUs; otherwise the first one that divides.
static const int kAuto[4] = {0, 1, 2, 3};

int choose_gateup_cfg(int T, int d, int F, int P, int swiglu) {
    const int64_t ngu = swiglu ? 2LL * F : (int64_t)F;
    int fallback = -1;
    for (int c : kAuto) {
        if (ngu % kCfgs[c].bm || d % 64) continue;
        const int64_t wgs = (int64_t)P * (ngu / kCfgs[c].bm) * cdiv(T, kCfgs[c].bn);
        if (fallback < 0) fallback = c;
        if (wgs >= 256) return c;
    }
    return fallback;
}

int choose_down_split(int T, int d, int P, int cfg) {
    if (cfg != 0 || d % 256) return 1;
    const int64_t tiles = (int64_t)(d / 256) * cdiv(T, 256);
    int best = 1;
    for (int s = 2; s <= P; ++s)                        // the largest divisor of P that keeps one round
        if (P % s == 0 && tiles * s <= 256) best = s;
    return best;
}

int64_t down_split_bytes(int64_t T_max, int d, int P) {
    int64_t most = 0;
    for (int64_t t = 256; t < T_max + 256; t += 256) {
        const int64_t T = t < T_max ? t : T_max;
        const int s = choose_down_split((int)T, d, P, 0);
        if (s > 1 && s * T * d * 4 > most) most = s * T * d * 4;
    }
    return most;
}

int choose_down_cfg(int T, int d, int F, int P) {
    int fallback = -1;
    for (int c : kAuto) {
        if (d % kCfgs[c].bm || F % 64) continue;
        const int64_t wgs = (d / kCfgs[c].bm) * cdiv(T, kCfgs[c].bn) * choose_down_split(T, d, P, c);
        if (fallback < 0) fallback = c;
        if (wgs >= 256) return c;
    }
    return fallback;
}

template <int BM, int BN, int WM, int WN>
static hipError_t gateup_go(const Bf16Args& a, hipStream_t st) {
    const int ngu = a.swiglu ? 2 * a.F : a.F;
    const int n_ft_shard = ngu / BM;
    const int n_tt = (int)cdiv(a.T, BN);
    const dim3 grid((unsigned)(a.P * n_ft_shard * n_tt));
    if (a.swiglu)
        hipLaunchKernelGGL((gateup_tiled<BM, BN, WM, WN, 1>), grid, dim3(WM * WN * 64), 0, st, a, n_ft_shard, n_tt);
    else
        hipLaunchKernelGGL((gateup_tiled<BM, BN, WM, WN, 2>), grid, dim3(WM * WN * 64), 0, st, a, n_ft_shard, n_tt);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t down_go(const Bf16Args& a, hipStream_t st) {
    const int n_ft = a.d / BM;
    const int n_tt = (int)cdiv(a.T, BN);
    hipLaunchKernelGGL((down_tiled<BM, BN, WM, WN>), dim3((unsigned)(n_ft * n_tt)), dim3(WM * WN * 64), 0, st,
                       a, n_ft, n_tt);
    return hipGetLastError();
}

hipError_t launch_gateup_tiled(const Bf16Args& a, int cfg, hipStream_t st) {
    switch (cfg) {
        case 0: {
            const int ngu = a.swiglu ? 2 * a.F : a.F;
            const int n_ft_shard = ngu / 256, n_tt = (int)cdiv(a.T, 256);
            const dim3 grid((unsigned)(a.P * n_ft_shard * n_tt));
            // buffer offsets are 32-bit: X (T x d bf16) and one stage's weight
            // slab (8 rows of 32 x d-element blocks) must each span < 2^31 bytes
            const bool buf = (int64_t)a.T * a.d * 2 < (int64_t(1) << 31) && (int64_t)a.d * 512 < (int64_t(1) << 31);
            const bool blk = a.nbt > 0;
            // raster groups sized so that the token slabs the eight XCDs'
            // current groups stream (8 x GT x 256 rows x d bf16) take at most
            // half of the 256 MB last-level cache: GT = 8 at d = 4096, 4 at
            // d = 8192 (measured: 70B long gate/up -2.7 % against 8, Llama
            // shape unchanged)
            Bf16Args b = a;
            b.gt = std::max(2, std::min(8, 32768 / a.d));
#define TSP_GU(ACT, BUF, BLK)                                                                             \
    do {                                                                                                  \
        if (a.save) hipLaunchKernelGGL((gateup_w16<ACT, BUF, BLK, true>), grid, dim3(256), 0, st, b, n_ft_shard, n_tt); \
        else hipLaunchKernelGGL((gateup_w16<ACT, BUF, BLK, false>), grid, dim3(256), 0, st, b, n_ft_shard, n_tt);     \
    } while (0)
            if (a.swiglu) {
                if (buf) { if (blk) TSP_GU(1, true, true); else TSP_GU(1, true, false); }
                else { if (blk) TSP_GU(1, false, true); else TSP_GU(1, false, false); }
            } else {
                if (buf) { if (blk) TSP_GU(2, true, true); else TSP_GU(2, true, false); }
                else { if (blk) TSP_GU(2, false, true); else TSP_GU(2, false, false); }
            }
#undef TSP_GU
            return hipGetLastError();
        }
        case 1: if (a.nbt || a.save) return hipErrorInvalidValue; return gateup_go<256, 128, 4, 2>(a, st);
        case 2: if (a.nbt || a.save) return hipErrorInvalidValue; return gateup_go<128, 128, 2, 2>(a, st);
        case 3: if (a.nbt || a.save) return hipErrorInvalidValue; return gateup_go<64, 128, 1, 4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down_tiled(const Bf16Args& a, int cfg, int split, hipStream_t st) {
    if (split > 1 && (cfg != 0 || a.P % split || !a.part)) return hipErrorInvalidValue;
    switch (cfg) {
        case 0: {
            const int n_ft = a.d / 256, n_tt = (int)cdiv(a.T, 256);
            const dim3 grid((unsigned)(n_ft * n_tt * split));
            // buffer offsets are 32-bit: one stage's weight slab (8 rows of
            // 32 x F-element blocks) and the operand H must each span < 2^31
            // bytes from their resource bases (blocked H: one column block of
            // nbt 1 KiB token blocks; row-major H: T x f)
            const bool buf = (int64_t)a.F * 512 < (int64_t(1) << 31) &&
                             (a.nbt ? (int64_t)a.nbt * 1024 : (int64_t)a.T * a.f * 2) < (int64_t(1) << 31);
            // raster groups of 4 token tiles (measured against 8: Llama down
            // -0.7 %, GeLU -1.7 %, 70B long -1.6 %)
            Bf16Args b = a;
            b.gt = 4;
#define TSP_DN(BLK, BUF) hipLaunchKernelGGL((down_w16<BLK, BUF>), grid, dim3(256), 0, st, b, n_ft, n_tt, split)
            if (a.nbt) { if (buf) TSP_DN(true, true); else TSP_DN(true, false); }
            else { if (buf) TSP_DN(false, true); else TSP_DN(false, false); }
#undef TSP_DN
            return hipGetLastError();
        }
        case 1: if (a.nbt) return hipErrorInvalidValue; return down_go<256, 128, 4, 2>(a, st);
        case 2: if (a.nbt) return hipErrorInvalidValue; return down_go<128, 128, 2, 2>(a, st);
        case 3: if (a.nbt) return hipErrorInvalidValue; return down_go<64, 128, 1, 4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce_partials(const float* part, int split, int64_t n, float* y, hipStream_t st) {
    const int64_t n4 = n / 4;                           // n = T * d, d a multiple of 64
    const int64_t blocks = std::min<int64_t>(cdiv(n4, 256), 4096);
    hipLaunchKernelGGL(reduce_partials, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(part), split, n4, reinterpret_cast<float4*>(y));
    return hipGetLastError();
}

}  // namespace tsp
