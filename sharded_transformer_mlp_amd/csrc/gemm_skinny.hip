// Skinny-T (T <= 32) weight-streaming kernels of the sharded MLP (gfx950).
//
// With at most 32 tokens every weight byte is used for at most 32 tokens, so
// the block is bound by reading the packed weights from HBM once. The packed
// 32 x 16 fragment blocks are contiguous 1 KiB pieces, so each wave load is a
// fully coalesced 16 bytes per lane; the tokens (one 32-column MFMA block,
// zero past T) come from L2. The MFMA is v_mfma_f32_32x32x16_bf16.
//
// skinny_gateup: one workgroup per 32 hidden columns of one shard (records
//   and the hidden columns they produce are both stored in ring order). Its
//   waves split the model dimension, each keeps fp32 gate and up
//   accumulators, the partial sums are added in LDS in wave order, and wave
//   0 applies the activation and writes the 32 hidden bf16 values of every
//   token straight into the MFMA token-fragment order the down product
//   reads (see below).
// skinny_down: one workgroup per 32 output features. The reduction runs over
//   all shards in ring order, flattened to one index range that the waves
//   split into consecutive pieces; the pieces are added in wave order, which
//   is ring order, and the fp32 result goes straight to Y.
//
// Skinny hidden-activation layout (library workspace): for every 16 hidden
// indices (ring-step order) one 1 KiB fragment block, lane l holding token
// l % 32 and hidden indices 8 (l / 32) .. + 7; so the down product loads its
// token operand with one contiguous 16-byte-per-lane access, like a weight
// block. Slots of tokens >= T are never written; they only feed output
// columns that are not stored.
#include "common.h"
#include "launch.h"

namespace tsp {

constexpr int SKG_NW = 8;      // waves per gate/up workgroup
constexpr int SKD_NW = 16;     // waves per down workgroup
constexpr int SK_U = 4;        // fragment blocks in flight per wave per operand

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Weight fragments are read exactly once per forward: nontemporal loads keep
// them from displacing the tokens / hidden activations in the caches (and
// stream HBM measurably faster than plain loads on this part).
__device__ __forceinline__ bf16x8 load_weight_frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// Token operand: lane l supplies token l % 32, reduction indices 8 * (l / 32) .. + 7.
__device__ __forceinline__ bf16x8 token_frag(const uint16_t* __restrict__ src, int ld, int64_t koff,
                                             int lane, int T) {
    const int tok = lane & 31;
    if (tok < T) return load_frag(src + (int64_t)tok * ld + koff + (lane >> 5) * 8);
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
}

template <int ACT>
__global__ __launch_bounds__(SKG_NW * 64) void skinny_gateup(Bf16Args a) {
    constexpr int NACC = ACT == 1 ? 2 : 1;              // gate and up, or A only
    __shared__ f32x16 red[SKG_NW][NACC][64];
    const int groups = a.F >> 5;                       // 32-column hidden groups per shard
    const int s = blockIdx.x / groups;                  // ring step = packed record
    const int grp = blockIdx.x - s * groups;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kb_total = a.d >> 4;
    const int kb_per = kb_total / SKG_NW;
    const int kb0 = w * kb_per;
    const int64_t rs = (int64_t)kb_total * 512;        // elements per 32-feature row of blocks
    const uint16_t* rec = a.packed + (int64_t)s * a.shard_elems;
    // SwiGLU: gate block 2*grp, up block 2*grp + 1; GeLU: block grp of A.
    const uint16_t* pg = rec + (ACT == 1 ? (int64_t)(2 * grp) * rs : (int64_t)grp * rs) + lane * 8;
    const uint16_t* pu = pg + rs;

    f32x16 acc[NACC];
#pragma unroll
    for (int c = 0; c < NACC; ++c) acc[c] = zero16();
    for (int kb = kb0; kb < kb0 + kb_per; kb += SK_U) {
        bf16x8 wv[NACC][SK_U], xv[SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            wv[0][u] = load_weight_frag(pg + (int64_t)(kb + u) * 512);
            if (NACC == 2) wv[NACC - 1][u] = load_weight_frag(pu + (int64_t)(kb + u) * 512);
            xv[u] = token_frag(a.x, a.d, (int64_t)(kb + u) * 16, lane, a.T);
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u)
#pragma unroll
            for (int c = 0; c < NACC; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[c][u], xv[u], acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < NACC; ++c) red[w][c][lane] = acc[c];
    __syncthreads();
    if (w == 0) {
        f32x16 sum[NACC];
#pragma unroll
        for (int c = 0; c < NACC; ++c) {
            sum[c] = red[0][c][lane];
#pragma unroll
            for (int i = 1; i < SKG_NW; ++i) sum[c] += red[i][c][lane];
        }
        const f32x16 g = sum[0], u = sum[NACC - 1];
        const int tok = lane & 31, h = lane >> 5;
        if (tok < a.T) {
            // this lane holds hidden 8 q + 4 h + r (q, r = 0..3) of the group:
            // fragment block 2 q' + q / 2 of the group (q' = group), chunk q % 2,
            // elements 4 h .. 4 h + 3 of that chunk for token tok
            const int64_t kb_base = ((int64_t)s * a.F + grp * 32) >> 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint2 v;
                if (ACT == 1)
                    v = pack4_bf16(silu_f(g[4 * q]) * u[4 * q], silu_f(g[4 * q + 1]) * u[4 * q + 1],
                                   silu_f(g[4 * q + 2]) * u[4 * q + 2], silu_f(g[4 * q + 3]) * u[4 * q + 3]);
                else
                    v = pack4_bf16(gelu_tanh_f(g[4 * q]), gelu_tanh_f(g[4 * q + 1]),
                                   gelu_tanh_f(g[4 * q + 2]), gelu_tanh_f(g[4 * q + 3]));
                uint16_t* blk = a.h + (kb_base + (q >> 1)) * 512;
                *reinterpret_cast<uint2*>(blk + ((q & 1) * 32 + tok) * 8 + 4 * h) = v;
            }
        }
    }
}

__global__ __launch_bounds__(SKD_NW * 64) void skinny_down(Bf16Args a) {
    __shared__ f32x16 red[SKD_NW][64];
    const int nb = blockIdx.x;                          // 32 output features
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kbF = a.F >> 4;                           // fragment blocks per shard
    const int kb_total = a.P * kbF;                     // flattened over the ring
    const int kb_per = kb_total / SKD_NW;
    const int kb0 = w * kb_per;
    const int64_t rs = (int64_t)kbF * 512;
    const uint16_t* base = a.packed + a.down_off + (int64_t)nb * rs + lane * 8;

    f32x16 acc = zero16();
    for (int kb = kb0; kb < kb0 + kb_per; kb += SK_U) {
        bf16x8 wv[SK_U], hv[SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int q = kb + u;                       // records and H are in ring order
            const int k = q / kbF, lk = q - k * kbF;
            wv[u] = load_weight_frag(base + (int64_t)k * a.shard_elems + (int64_t)lk * 512);
            hv[u] = load_frag(a.h + (int64_t)q * 512 + lane * 8);     // fragment-ordered H
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[u], hv[u], acc, 0, 0, 0);
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        f32x16 y = red[0][lane];
#pragma unroll
        for (int i = 1; i < SKD_NW; ++i) y += red[i][lane];
        const int tok = lane & 31;
        if (tok < a.T) {
            float* yrow = a.y + (int64_t)tok * a.d + nb * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(yrow + 8 * q) =
                    make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
        }
    }
}

bool skinny_supported(int d, int F, int P) {
    // every wave gets a whole number of SK_U-block groups
    const int64_t kb_gu = d / 16, kb_dn = (int64_t)P * (F / 16);
    return d % 64 == 0 && F % 64 == 0 && kb_gu % (SKG_NW * SK_U) == 0 && kb_dn % (SKD_NW * SK_U) == 0;
}

hipError_t launch_gateup_skinny(const Bf16Args& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.P * (a.F / 32)));
    if (a.swiglu)
        hipLaunchKernelGGL(skinny_gateup<1>, grid, dim3(SKG_NW * 64), 0, st, a);
    else
        hipLaunchKernelGGL(skinny_gateup<2>, grid, dim3(SKG_NW * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_down_skinny(const Bf16Args& a, hipStream_t st) {
    hipLaunchKernelGGL(skinny_down, dim3((unsigned)(a.d / 32)), dim3(SKD_NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace tsp
