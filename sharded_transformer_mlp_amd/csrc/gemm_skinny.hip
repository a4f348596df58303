// Skinny-T (T <= 16) weight-streaming kernels of the sharded MLP (gfx950).
//
// With at most 16 tokens every weight byte is used for at most 16 tokens, so
// the block is bound by reading the packed weights from HBM once. The packed
// 16 x 32 fragment blocks are contiguous 1 KiB pieces, so each wave load is a
// fully coalesced 16 bytes per lane, and the tokens (one 16-column MFMA block,
// zero-padded past T) come from L2.
//
// skinny_gateup: one workgroup per 16 hidden columns of one shard (records
//   and the hidden columns they produce are both stored in ring order). Its
//   NW waves split the model dimension, each keeps fp32 gate and up
//   accumulators, the partial sums are added in LDS in wave
//   order, and wave 0 applies the activation and writes 16 tokens x 16
//   hidden bf16 values.
// skinny_down: one workgroup per 16 output features. The reduction runs over
//   all shards in ring order, flattened to one index range that the NW waves
//   split into consecutive pieces; the pieces are added in wave order, which
//   is ring order, and the fp32 result goes straight to Y.
#include "common.h"
#include "launch.h"

namespace tsp {

constexpr int SK_NW = 8;       // waves per workgroup
constexpr int SK_U = 4;        // fragment blocks in flight per wave per operand

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 token_frag(const uint16_t* __restrict__ src, int ld, int64_t koff,
                                             int lane, int T) {
    const int tok = lane & 15;
    if (tok < T) return load_frag(src + (int64_t)tok * ld + koff + (lane >> 4) * 8);
    return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

template <int ACT>
__global__ __launch_bounds__(SK_NW * 64) void skinny_gateup(Bf16Args a) {
    __shared__ f32x4 red[SK_NW][2][64];
    const int groups = a.F >> 4;                       // 16-column hidden groups per shard
    const int s = blockIdx.x / groups;                  // ring step = packed record
    const int grp = blockIdx.x - s * groups;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kb_total = a.d >> 5;
    const int kb_per = kb_total / SK_NW;
    const int kb0 = w * kb_per;
    const int64_t rs = (int64_t)kb_total * 512;        // elements per 16-feature row of blocks
    const uint16_t* rec = a.packed + (int64_t)s * a.shard_elems;
    // SwiGLU: gate block 2*grp, up block 2*grp + 1; GeLU: block grp of A.
    const uint16_t* pg = rec + (ACT == 1 ? (int64_t)(2 * grp) * rs : (int64_t)grp * rs) + lane * 8;
    const uint16_t* pu = pg + rs;

    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    for (int kb = kb0; kb < kb0 + kb_per; kb += SK_U) {
        bf16x8 wg[SK_U], wu[SK_U], xv[SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            wg[u] = load_frag(pg + (int64_t)(kb + u) * 512);
            if (ACT == 1) wu[u] = load_frag(pu + (int64_t)(kb + u) * 512);
            xv[u] = token_frag(a.x, a.d, (int64_t)(kb + u) * 32, lane, a.T);
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg[u], xv[u], ag, 0, 0, 0);
            if (ACT == 1) au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wu[u], xv[u], au, 0, 0, 0);
        }
    }
    red[w][0][lane] = ag;
    red[w][1][lane] = au;
    __syncthreads();
    if (w == 0) {
        f32x4 g = red[0][0][lane], u = red[0][1][lane];
#pragma unroll
        for (int i = 1; i < SK_NW; ++i) {
            g += red[i][0][lane];
            u += red[i][1][lane];
        }
        const int tok = lane & 15;
        if (tok < a.T) {
            const int hcol = s * a.F + grp * 16 + (lane >> 4) * 4;
            uint2 v;
            if (ACT == 1)
                v = pack4_bf16(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1], silu_f(g[2]) * u[2],
                               silu_f(g[3]) * u[3]);
            else
                v = pack4_bf16(gelu_tanh_f(g[0]), gelu_tanh_f(g[1]), gelu_tanh_f(g[2]),
                               gelu_tanh_f(g[3]));
            *reinterpret_cast<uint2*>(a.h + (int64_t)tok * a.f + hcol) = v;
        }
    }
}

__global__ __launch_bounds__(SK_NW * 64) void skinny_down(Bf16Args a) {
    __shared__ f32x4 red[SK_NW][64];
    const int nb = blockIdx.x;                          // 16 output features
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kbF = a.F >> 5;                           // fragment blocks per shard
    const int kb_total = a.P * kbF;                     // flattened over the ring
    const int kb_per = kb_total / SK_NW;
    const int kb0 = w * kb_per;
    const int64_t rs = (int64_t)kbF * 512;
    const uint16_t* base = a.packed + a.down_off + (int64_t)nb * rs + lane * 8;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb = kb0; kb < kb0 + kb_per; kb += SK_U) {
        bf16x8 wv[SK_U], hv[SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int q = kb + u;                       // records and H are in ring order
            const int k = q / kbF, lk = q - k * kbF;
            wv[u] = load_frag(base + (int64_t)k * a.shard_elems + (int64_t)lk * 512);
            hv[u] = token_frag(a.h, a.f, (int64_t)q * 32, lane, a.T);
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[u], hv[u], acc, 0, 0, 0);
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        f32x4 y = red[0][lane];
#pragma unroll
        for (int i = 1; i < SK_NW; ++i) y += red[i][lane];
        const int tok = lane & 15;
        if (tok < a.T) {
            const int n = nb * 16 + (lane >> 4) * 4;
            *reinterpret_cast<float4*>(a.y + (int64_t)tok * a.d + n) = make_float4(y[0], y[1], y[2], y[3]);
        }
    }
}

bool skinny_supported(int d, int F, int P) {
    // every wave gets a whole number of SK_U-block groups
    const int64_t kb_gu = d / 32, kb_dn = (int64_t)P * (F / 32);
    return d % 64 == 0 && F % 64 == 0 && kb_gu % (SK_NW * SK_U) == 0 && kb_dn % (SK_NW * SK_U) == 0;
}

hipError_t launch_gateup_skinny(const Bf16Args& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.P * (a.F / 16)));
    if (a.swiglu)
        hipLaunchKernelGGL(skinny_gateup<1>, grid, dim3(SK_NW * 64), 0, st, a);
    else
        hipLaunchKernelGGL(skinny_gateup<2>, grid, dim3(SK_NW * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_down_skinny(const Bf16Args& a, hipStream_t st) {
    hipLaunchKernelGGL(skinny_down, dim3((unsigned)(a.d / 16)), dim3(SK_NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace tsp
