// Tiled bf16 MFMA kernels of the sharded MLP (gfx950).
//
// Both products run with the weights as the MFMA A operand (rows = output
// features) and the tokens as the B operand (columns = tokens), using
// v_mfma_f32_16x16x32_bf16. Each lane then holds 4 consecutive output
// features of one token, so the epilogue writes H (bf16) and Y (fp32) rows
// straight from registers.
//
// gateup_tiled: H[:, cols of shard s] = act(X . W_s) for every shard, the
//   SwiGLU or GeLU epilogue applied in registers ("Tensor Parallelism:
//   Splitting the Math", section "Why the column-then-row split": the
//   nonlinearity is exact on a shard's own columns). Tiles of the shard
//   visited at ring step k are dispatched before those of step k + 1.
// down_tiled:   Y = sum_k H_{order[k]} . Wd_{order[k]}; the reduction loop
//   walks the shards in ring order and keeps the fp32 Y tile in registers
//   for the whole walk, so Y is written once ("Folding Tensor and Sequence
//   Parallelism ...", Abstract: partial outputs accumulate locally).
//
// Main loop: a BM x 64 slab of packed weights and a BN x 64 slab of tokens
// per step, staged through registers into double-buffered LDS laid out in
// fragment blocks (1 KiB per 16 rows x 32 reduction indices, lane-ordered),
// so every LDS read of an operand fragment is one contiguous 16-byte-per-lane
// access. One barrier per step.
#include "common.h"
#include "launch.h"

namespace tsp {

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;            // threads
    static constexpr int TM = BM / WM / 16;             // MFMA blocks per wave along features
    static constexpr int TN = BN / WN / 16;             // MFMA blocks per wave along tokens
    static constexpr int CA = BM * 8 / NT;              // 16-byte chunks per thread per step (A)
    static constexpr int CB = BN * 8 / NT;              // (B)
    static constexpr int A_ELEMS = BM * 64;             // bf16 elements per stage
    static constexpr int B_ELEMS = BN * 64;
    static constexpr int STAGE = A_ELEMS + B_ELEMS;
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(CA * NT == BM * 8 && CB * NT == BN * 8, "loader split");
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

template <class C>
__device__ __forceinline__ void load_a(const uint16_t* __restrict__ a_base, int64_t a_rs,
                                       uint4 (&ra)[C::CA]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
        const int q = i * C::NT + tid;
        const int blk = q >> 6, lane = q & 63;
        ra[i] = *reinterpret_cast<const uint4*>(a_base + (blk >> 1) * a_rs + (blk & 1) * 512 + lane * 8);
    }
}

template <class C>
__device__ __forceinline__ void load_b(const uint16_t* __restrict__ b_src, int ldb, int64_t b_koff,
                                       int t0, int T, uint4 (&rb)[C::CB]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
        const int q = i * C::NT + tid;
        const int blk = q >> 6, lane = q & 63;
        const int tok = t0 + (blk >> 1) * 16 + (lane & 15);
        if (tok < T) {
            rb[i] = *reinterpret_cast<const uint4*>(b_src + (int64_t)tok * ldb + b_koff +
                                                   (blk & 1) * 32 + (lane >> 4) * 8);
        } else {
            rb[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

template <class C>
__device__ __forceinline__ void store_stage(uint16_t* lds_stage, const uint4 (&ra)[C::CA],
                                            const uint4 (&rb)[C::CB]) {
    uint4* as = reinterpret_cast<uint4*>(lds_stage);
    uint4* bs = reinterpret_cast<uint4*>(lds_stage + C::A_ELEMS);
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::CA; ++i) as[i * C::NT + tid] = ra[i];
#pragma unroll
    for (int i = 0; i < C::CB; ++i) bs[i * C::NT + tid] = rb[i];
}

template <class C>
__device__ __forceinline__ void compute_stage(const uint16_t* lds_stage, f32x4 (&acc)[C::TM][C::TN],
                                              int wm, int wn, int lane) {
    const bf16x8* as = reinterpret_cast<const bf16x8*>(lds_stage);
    const bf16x8* bs = reinterpret_cast<const bf16x8*>(lds_stage + C::A_ELEMS);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8 af[C::TM], bv[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) af[i] = as[((wm * C::TM + i) * 2 + kk) * 64 + lane];
#pragma unroll
        for (int j = 0; j < C::TN; ++j) bv[j] = bs[((wn * C::TN + j) * 2 + kk) * 64 + lane];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bv[j], acc[i][j], 0, 0, 0);
    }
}

// act: 1 = SwiGLU (packed blocks alternate gate / up), 2 = GeLU (tanh form)
template <int BM, int BN, int WM, int WN, int ACT>
__global__ __launch_bounds__(WM * WN * 64) void gateup_tiled(Bf16Args a, int n_ft_shard, int n_tt) {
    using C = TileCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];

    int ttile, flin;
    raster(xcd_remap(blockIdx.x, gridDim.x), a.P * n_ft_shard, n_tt, ttile, flin);
    const int step = flin / n_ft_shard;                 // ring step
    const int ftile = flin - step * n_ft_shard;
    const int s = a.order[step];                        // shard held at that step
    const int kblocks = a.d >> 5;
    const int64_t a_rs = (int64_t)kblocks * 512;
    const uint16_t* a_tile = a.packed + (int64_t)s * a.shard_elems + (int64_t)(ftile * (BM / 16)) * a_rs;
    const int t0 = ttile * BN;
    const int ksteps = a.d >> 6;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int wm = wid / WN, wn = wid % WN;

    f32x4 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[C::CA], rb[C::CB];
    load_a<C>(a_tile, a_rs, ra);
    load_b<C>(a.x, a.d, 0, t0, a.T, rb);
    store_stage<C>(lds, ra, rb);
    __syncthreads();
    for (int t = 0; t < ksteps; ++t) {
        const int cur = t & 1;
        if (t + 1 < ksteps) {
            load_a<C>(a_tile + (int64_t)(t + 1) * 1024, a_rs, ra);
            load_b<C>(a.x, a.d, (int64_t)(t + 1) * 64, t0, a.T, rb);
        }
        compute_stage<C>(lds + cur * C::STAGE, acc, wm, wn, lane);
        if (t + 1 < ksteps) store_stage<C>(lds + (cur ^ 1) * C::STAGE, ra, rb);
        __syncthreads();
    }

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
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::STAGE];

    int ttile, ftile;
    raster(xcd_remap(blockIdx.x, gridDim.x), n_ft, n_tt, ttile, ftile);
    const int kbF = a.F >> 5;
    const int spp = a.F >> 6;                           // steps per shard
    const int ksteps = a.P * spp;
    const int64_t a_rs = (int64_t)kbF * 512;
    const uint16_t* a_ft = a.packed + a.down_off + (int64_t)(ftile * (BM / 16)) * a_rs;
    const int t0 = ttile * BN;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int wm = wid / WN, wn = wid % WN;

    f32x4 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[C::CA], rb[C::CB];
    {
        const int s = a.order[0];
        load_a<C>(a_ft + (int64_t)s * a.shard_elems, a_rs, ra);
        load_b<C>(a.h, a.f, (int64_t)s * a.F, t0, a.T, rb);
    }
    store_stage<C>(lds, ra, rb);
    __syncthreads();
    for (int t = 0; t < ksteps; ++t) {
        const int cur = t & 1;
        if (t + 1 < ksteps) {
            const int k = (t + 1) / spp, ls = (t + 1) - k * spp;
            const int s = a.order[k];
            load_a<C>(a_ft + (int64_t)s * a.shard_elems + (int64_t)ls * 1024, a_rs, ra);
            load_b<C>(a.h, a.f, (int64_t)s * a.F + ls * 64, t0, a.T, rb);
        }
        compute_stage<C>(lds + cur * C::STAGE, acc, wm, wn, lane);
        if (t + 1 < ksteps) store_stage<C>(lds + (cur ^ 1) * C::STAGE, ra, rb);
        __syncthreads();
    }

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
