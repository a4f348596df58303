// Tiled bf16 MFMA kernels of the sharded MLP (gfx950).
//
// Both products run with the weights as the MFMA A operand (rows = output
// features) and the tokens as the B operand (columns = tokens), using
// v_mfma_f32_16x16x32_bf16. Each lane then holds 4 consecutive output
// features of one token, so the epilogue writes H (bf16) and Y (fp32) rows
// straight from registers.
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
// Main loop: 32 reduction indices per stage, a 4-deep LDS ring filled by
// global_load_lds_dwordx4 (global memory straight into LDS, no register
// staging). Loads for stage t + 3 are issued right after the barrier of
// stage t, so each stage's loads have three stages of MFMA work to land. LDS
// is laid out in fragment blocks (1 KiB per 16 rows x 32 reduction indices,
// lane-ordered), so every operand fragment read is one contiguous
// 16-byte-per-lane access.
#include "common.h"
#include "launch.h"

namespace tsp {

#define TSP_LDS __attribute__((address_space(3)))

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN;                   // waves
    static constexpr int NT = NW * 64;                   // threads
    static constexpr int TM = BM / WM / 16;              // MFMA blocks per wave along features
    static constexpr int TN = BN / WN / 16;              // MFMA blocks per wave along tokens
    static constexpr int A_BLK = BM / 16;                // 1 KiB fragment blocks per stage (A)
    static constexpr int B_BLK = BN / 16;                // (B)
    static constexpr int LOADS = (A_BLK + B_BLK) / NW;   // DMA loads per wave per stage
    static constexpr int STAGE = (A_BLK + B_BLK) * 512;  // bf16 elements per stage (32-deep)
    static constexpr int NS = 4;                         // stages in the LDS ring
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(LOADS * NW == A_BLK + B_BLK, "loader split");
    static_assert(NS * STAGE * 2 <= 160 * 1024, "LDS");
};

// Token-tile-grouped raster over a (tokens x features) tile grid: GT token
// tiles share each feature tile, consecutive ids walk the token tiles first.
__device__ inline void raster(int L, int n_f, int n_t, int& ttile, int& flin) {
    constexpr int GT = 8;
    const int group = L / (GT * n_f);
    const int first = group * GT;
    const int gt = min(GT, n_t - first);
    const int rem = L - group * GT * n_f;
    ttile = first + rem % gt;
    flin = rem / gt;
}

// One pipeline stage = 32 reduction indices of the A slab (BM packed weight
// rows, 16-row fragment blocks) and the B slab (BN tokens). Each wave moves
// LOADS whole 1 KiB blocks with global_load_lds_dwordx4: the 64 lanes' 16-byte
// pieces land contiguously in LDS, already in fragment order. Token rows past
// T are clamped to row T - 1 (their outputs are never stored).
template <class C>
__device__ __forceinline__ void issue_stage(uint16_t* lds_stage, const uint16_t* __restrict__ a_base,
                                            int64_t a_rs, const uint16_t* __restrict__ b_src, int ldb,
                                            int64_t b_koff, int t0, int T, int w, int lane) {
#pragma unroll
    for (int r = 0; r < C::LOADS; ++r) {
        const int b = r * C::NW + w;                     // wave-uniform block id
        const uint16_t* g;
        if (b < C::A_BLK) {
            g = a_base + b * a_rs + lane * 8;
        } else {
            const int tok = min(t0 + (b - C::A_BLK) * 16 + (lane & 15), T - 1);
            g = b_src + (int64_t)tok * ldb + b_koff + (lane >> 4) * 8;
        }
        __builtin_amdgcn_global_load_lds(g, (TSP_LDS void*)(lds_stage + b * 512), 16, 0, 0);
    }
}

// Wait until at most `newer` stages of this wave's DMA loads are outstanding.
template <class C>
__device__ __forceinline__ void wait_stages(int newer) {
    // s_waitcnt with vmcnt = newer * LOADS, expcnt / lgkmcnt left at their maximum
#define TSP_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
    if (newer >= 3) TSP_VMCNT(3 * C::LOADS);
    else if (newer == 2) TSP_VMCNT(2 * C::LOADS);
    else if (newer == 1) TSP_VMCNT(C::LOADS);
    else TSP_VMCNT(0);
#undef TSP_VMCNT
}

// Workgroup barrier that orders LDS traffic without waiting for the DMA
// loads still in flight for later stages (__syncthreads would drain them).
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <class C>
__device__ __forceinline__ void read_frags(const uint16_t* lds_stage, bf16x8 (&af)[C::TM],
                                           bf16x8 (&bv)[C::TN], int wm, int wn, int lane) {
    const bf16x8* as = reinterpret_cast<const bf16x8*>(lds_stage);
    const bf16x8* bs = reinterpret_cast<const bf16x8*>(lds_stage + C::A_BLK * 512);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) af[i] = as[(wm * C::TM + i) * 64 + lane];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) bv[j] = bs[(wn * C::TN + j) * 64 + lane];
}

template <class C>
__device__ __forceinline__ void mfma_stage(f32x4 (&acc)[C::TM][C::TN], const bf16x8 (&af)[C::TM],
                                           const bf16x8 (&bv)[C::TN]) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bv[j], acc[i][j], 0, 0, 0);
}

// The reduction loop shared by both kernels. `src(t, a_base, b_koff)` gives
// step t's A slab start and B reduction offset (32 indices per step).
//
// Ping-pong schedule: the waves form two groups (waves 0..NW/2-1 and the
// rest), one wave of each group per SIMD. Each step t is a memory phase M(t)
// (issue the DMA loads of stage t + 3, read stage t's fragments from LDS) and
// a compute phase C(t) (the MFMAs). Group 1 runs one phase behind group 0,
// and every phase boundary is a workgroup barrier, so on each SIMD one wave
// computes while the other does its memory work.
//
// Barrier b_{2t} opens group 0's M(t) (group 1's C(t-1)); b_{2t+1} opens
// group 0's C(t) (group 1's M(t)). Every wave makes its own stage-t loads
// complete before b_{2t}, so stage t is visible to both groups' M(t). The
// DMA of stage t + 3 goes into stage t - 1's buffer, whose last reader
// (group 1's M(t-1), which drains its LDS reads before b_{2t}) is done.
template <class C, class Src>
__device__ __forceinline__ void mainloop(uint16_t* lds, f32x4 (&acc)[C::TM][C::TN], int ksteps,
                                         int64_t a_rs, const uint16_t* b_src, int ldb, int t0, int T,
                                         Src&& src) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / C::WN, wn = w % C::WN;
    const bool g1 = w >= C::NW / 2;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto issue = [&](int t) {
        const uint16_t* ab;
        int64_t bk;
        src(t, ab, bk);
        issue_stage<C>(lds + (t % C::NS) * C::STAGE, ab, a_rs, b_src, ldb, bk, t0, T, w, lane);
    };
    constexpr int AHEAD = C::NS - 1;                    // stages in flight ahead of the reader
    const int pro = min(AHEAD, ksteps);
    for (int t = 0; t < pro; ++t) issue(t);
    wait_stages<C>(pro - 1);                            // own stage-0 loads landed
    if (g1) stage_barrier();                            // b_0: group 1 sits out phase 0
    bf16x8 af[C::TM], bv[C::TN];
    for (int t = 0; t < ksteps; ++t) {
        stage_barrier();                                // g0: b_{2t}, g1: b_{2t+1}
        __builtin_amdgcn_sched_barrier(0);
        if (t + AHEAD < ksteps) issue(t + AHEAD);
        read_frags<C>(lds + (t % C::NS) * C::STAGE, af, bv, wm, wn, lane);
        __builtin_amdgcn_s_waitcnt((15 & 15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
        // stage t + 1 must be complete before b_{2t+2}: group 1 reaches it
        // at the end of this memory phase, group 0 after its compute phase
        const int newer = min(t + AHEAD, ksteps - 1) - (t + 1);
        if (g1) wait_stages<C>(newer);
        __builtin_amdgcn_sched_barrier(0);
        stage_barrier();                                // g0: b_{2t+1}, g1: b_{2t+2}
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        mfma_stage<C>(acc, af, bv);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        if (!g1) wait_stages<C>(newer);
    }
    if (!g1) stage_barrier();                           // b_{2K}: group 0 matches group 1's count
}

// act: 1 = SwiGLU (packed blocks alternate gate / up), 2 = GeLU (tanh form)
template <int BM, int BN, int WM, int WN, int ACT>
__global__ __launch_bounds__(WM * WN * 64) void gateup_tiled(Bf16Args a, int n_ft_shard, int n_tt) {
    using C = TileCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];

    int ttile, flin;
    raster(xcd_remap(blockIdx.x, gridDim.x), a.P * n_ft_shard, n_tt, ttile, flin);
    const int s = flin / n_ft_shard;                    // ring step = packed record
    const int ftile = flin - s * n_ft_shard;
    const int64_t a_rs = (int64_t)(a.d >> 5) * 512;     // elements per 16-row block row
    const uint16_t* a_tile = a.packed + (int64_t)s * a.shard_elems + (int64_t)(ftile * (BM / 16)) * a_rs;
    const int t0 = ttile * BN;

    f32x4 acc[C::TM][C::TN];
    mainloop<C>(lds, acc, a.d >> 5, a_rs, a.x, a.d, t0, a.T,
                [&](int t, const uint16_t*& ab, int64_t& bk) {
                    ab = a_tile + (int64_t)t * 512;
                    bk = (int64_t)t * 32;
                });

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    if constexpr (ACT == 1) {
#pragma unroll
        for (int p = 0; p < C::TM / 2; ++p) {
            const int gb = ftile * (BM / 16) + wm * C::TM + 2 * p;     // gate block (even)
            const int hcol = s * a.F + (gb >> 1) * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int tok = t0 + (wn * C::TN + j) * 16 + (lane & 15);
                if (tok < a.T) {
                    const f32x4 g = acc[2 * p][j], u = acc[2 * p + 1][j];
                    *reinterpret_cast<uint2*>(a.h + (int64_t)tok * a.f + hcol) =
                        pack4_bf16(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1],
                                   silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int hcol = s * a.F + (ftile * (BM / 16) + wm * C::TM + i) * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int tok = t0 + (wn * C::TN + j) * 16 + (lane & 15);
                if (tok < a.T) {
                    const f32x4 u = acc[i][j];
                    *reinterpret_cast<uint2*>(a.h + (int64_t)tok * a.f + hcol) =
                        pack4_bf16(gelu_tanh_f(u[0]), gelu_tanh_f(u[1]), gelu_tanh_f(u[2]),
                                   gelu_tanh_f(u[3]));
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void down_tiled(Bf16Args a, int n_ft, int n_tt) {
    using C = TileCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];

    int ttile, ftile;
    raster(xcd_remap(blockIdx.x, gridDim.x), n_ft, n_tt, ttile, ftile);
    const int spp = a.F >> 5;                           // steps per shard
    const int64_t a_rs = (int64_t)spp * 512;
    const uint16_t* a_ft = a.packed + a.down_off + (int64_t)(ftile * (BM / 16)) * a_rs;
    const int t0 = ttile * BN;

    f32x4 acc[C::TM][C::TN];
    // Reduction step t is local step t % spp of ring step t / spp; records
    // and H columns are both stored in ring order, so this is a linear walk.
    mainloop<C>(lds, acc, a.P * spp, a_rs, a.h, a.f, t0, a.T,
                [&](int t, const uint16_t*& ab, int64_t& bk) {
                    const int k = t / spp, ls = t - k * spp;
                    ab = a_ft + (int64_t)k * a.shard_elems + (int64_t)ls * 512;
                    bk = (int64_t)t * 32;
                });

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int n = ftile * BM + (wm * C::TM + i) * 16 + (lane >> 4) * 4;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int tok = t0 + (wn * C::TN + j) * 16 + (lane & 15);
            if (tok < a.T) {
                const f32x4 v = acc[i][j];
                *reinterpret_cast<float4*>(a.y + (int64_t)tok * a.d + n) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// ------------------------------------------------------------------ configs
// cfg: 0 = 256 x 256 (8 waves as 4 x 2), 1 = 256 x 128 (8 waves),
//      2 = 128 x 128 (4 waves as 2 x 2), 3 = 64 x 128 (4 waves as 1 x 4)
struct CfgDesc { int bm, bn; const char* name; };
static const CfgDesc kCfgs[4] = {
    {256, 256, "256x256"}, {256, 128, "256x128"}, {128, 128, "128x128"}, {64, 128, "64x128"}};

const char* tiled_cfg_name(int cfg) { return (cfg >= 0 && cfg < 4) ? kCfgs[cfg].name : "none"; }

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool gateup_cfg_fits(int cfg, int d, int F, int swiglu) {
    if (cfg < 0 || cfg >= 4) return false;
    const int64_t ngu = swiglu ? 2LL * F : (int64_t)F;
    return ngu % kCfgs[cfg].bm == 0 && d % 64 == 0;
}

bool down_cfg_fits(int cfg, int d, int F) {
    return cfg >= 0 && cfg < 4 && d % kCfgs[cfg].bm == 0 && F % 64 == 0;
}

int choose_gateup_cfg(int T, int d, int F, int P, int swiglu) {
    // Largest tile that divides the shard's packed width and still gives at
    // least one full wave of workgroups on 256 CUs; otherwise the largest
    // that divides.
    const int64_t ngu = swiglu ? 2LL * F : (int64_t)F;
    int fallback = -1;
    for (int c = 0; c < 4; ++c) {
        if (ngu % kCfgs[c].bm || d % 64) continue;
        const int64_t wgs = (int64_t)P * (ngu / kCfgs[c].bm) * cdiv(T, kCfgs[c].bn);
        if (fallback < 0) fallback = c;
        if (wgs >= 256) return c;
    }
    return fallback;
}

int choose_down_cfg(int T, int d, int F) {
    int fallback = -1;
    for (int c = 0; c < 4; ++c) {
        if (d % kCfgs[c].bm || F % 64) continue;
        const int64_t wgs = (d / kCfgs[c].bm) * cdiv(T, kCfgs[c].bn);
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
        case 0: return gateup_go<256, 256, 4, 2>(a, st);
        case 1: return gateup_go<256, 128, 4, 2>(a, st);
        case 2: return gateup_go<128, 128, 2, 2>(a, st);
        case 3: return gateup_go<64, 128, 1, 4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down_tiled(const Bf16Args& a, int cfg, hipStream_t st) {
    switch (cfg) {
        case 0: return down_go<256, 256, 4, 2>(a, st);
        case 1: return down_go<256, 128, 4, 2>(a, st);
        case 2: return down_go<128, 128, 2, 2>(a, st);
        case 3: return down_go<64, 128, 1, 4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tsp
