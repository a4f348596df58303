// Skinny-T (T <= 32) weight-streaming kernels of the sharded MLP (gfx950).
//
// With at most 32 tokens every weight byte is used for at most 32 tokens, so
// the block is bound by reading the packed weights from HBM once. The packed
// 32 x 16 fragment blocks are contiguous 1 KiB pieces, so each wave load is a
// fully coalesced 16 bytes per lane; the tokens (one 32-column MFMA block,
// zero past T) come from L2. The MFMA is v_mfma_f32_32x32x16_bf16.
//
// skinny_gateup: one workgroup per SK_G groups of 32 hidden columns of one
//   shard (records and the hidden columns they produce are both stored in
//   ring order), so each token fragment it loads feeds 2 * SK_G (SwiGLU) or
//   SK_G weight blocks. Its waves take the model dimension's fragment blocks
//   in an interleaved order (wave w: blocks w * SK_U + i * SKG_NW * SK_U ..),
//   so the workgroup reads each weight row front to back as one stream. Each
//   wave keeps fp32 accumulators, the partial sums are added in LDS in wave
//   order, and wave g applies the activation for group g and writes the 32
//   hidden bf16 values of every token straight into the MFMA token-fragment
//   order the down product reads (see below).
// skinny_down: one workgroup per 32 output features. The reduction runs over
//   all shards in ring order, flattened to one range of fragment blocks that
//   the waves take interleaved like the gate/up kernel; the per-wave partial
//   sums are added in wave order (a fixed order, so results are bitwise
//   reproducible) and the fp32 result goes straight to Y.
//
// Skinny hidden-activation layout (library workspace): for every 16 hidden
// indices (ring-step order) one 1 KiB fragment block, lane l holding token
// l % 32 and hidden indices 8 (l / 32) .. + 7; so the down product loads its
// token operand with one contiguous 16-byte-per-lane access, like a weight
// block. Slots of tokens >= T are never written nor read (those lanes feed a
// zero operand instead).
#include "common.h"
#include "launch.h"

namespace tsp {

constexpr int SKG_NW = 4;      // waves per gate/up workgroup
constexpr int SK_G = 2;        // 32-column hidden groups per gate/up workgroup
constexpr int SKD_NW = 16;     // waves per down workgroup
constexpr int SK_U = 4;        // fragment blocks in flight per wave per weight row

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
    constexpr int NR = SK_G * NACC;                     // 32-feature block rows per workgroup
    __shared__ f32x16 red[SKG_NW][NR][64];
    poison_lds(red, sizeof(red));
    const int wg_per_shard = (a.F >> 5) / SK_G;
    const int s = blockIdx.x / wg_per_shard;            // ring step = packed record
    const int grp0 = (blockIdx.x - s * wg_per_shard) * SK_G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kb_total = a.d >> 4;
    const int64_t rs = (int64_t)kb_total * 512;        // elements per 32-feature row of blocks
    // Block row grp * NACC + c holds group grp's gate (c = 0) / up (c = 1)
    // features for SwiGLU, or its A features for GeLU: the workgroup's NR rows
    // are consecutive.
    const uint16_t* p0 = a.packed + (int64_t)s * a.shard_elems + (int64_t)(grp0 * NACC) * rs + lane * 8;

    f32x16 acc[NR];
#pragma unroll
    for (int c = 0; c < NR; ++c) acc[c] = zero16();
    for (int kb = w * SK_U; kb < kb_total; kb += SKG_NW * SK_U) {
        bf16x8 wv[NR][SK_U], xv[SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
#pragma unroll
            for (int c = 0; c < NR; ++c) wv[c][u] = load_weight_frag(p0 + c * rs + (int64_t)(kb + u) * 512);
            xv[u] = token_frag(a.x, a.d, (int64_t)(kb + u) * 16, lane, a.T);
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u)
#pragma unroll
            for (int c = 0; c < NR; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[c][u], xv[u], acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < NR; ++c) red[w][c][lane] = acc[c];
    __syncthreads();
    for (int g = w; g < SK_G; g += SKG_NW) {
        const int grp = grp0 + g;
        f32x16 gs = red[0][g * NACC][lane], us = red[0][g * NACC + NACC - 1][lane];
#pragma unroll
        for (int i = 1; i < SKG_NW; ++i) {
            gs += red[i][g * NACC][lane];
            if (NACC == 2) us += red[i][g * NACC + 1][lane];
        }
        const int tok = lane & 31, h = lane >> 5;
        if (tok < a.T) {
            // this lane holds hidden 8 q + 4 h + r (q, r = 0..3) of the group:
            // fragment block q / 2 of the group, chunk q % 2, elements
            // 4 h .. 4 h + 3 of that chunk for token tok
            const int64_t kb_base = ((int64_t)s * a.F + grp * 32) >> 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint2 v;
                if (ACT == 1)
                    v = pack4_bf16(silu_f(gs[4 * q]) * us[4 * q], silu_f(gs[4 * q + 1]) * us[4 * q + 1],
                                   silu_f(gs[4 * q + 2]) * us[4 * q + 2], silu_f(gs[4 * q + 3]) * us[4 * q + 3]);
                else
                    v = pack4_bf16(gelu_tanh_f(gs[4 * q]), gelu_tanh_f(gs[4 * q + 1]),
                                   gelu_tanh_f(gs[4 * q + 2]), gelu_tanh_f(gs[4 * q + 3]));
                uint16_t* blk = a.h + (kb_base + (q >> 1)) * 512;
                *reinterpret_cast<uint2*>(blk + ((q & 1) * 32 + tok) * 8 + 4 * h) = v;
            }
        }
    }
}

__global__ __launch_bounds__(SKD_NW * 64) void skinny_down(Bf16Args a) {
    __shared__ f32x16 red[SKD_NW][64];
    poison_lds(red, sizeof(red));
    const int nb = blockIdx.x;                          // 32 output features
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kbF = a.F >> 4;                           // fragment blocks per shard
    const int kb_total = a.P * kbF;                     // flattened over the ring
    const int64_t rs = (int64_t)kbF * 512;
    const uint16_t* base = a.packed + a.down_off + (int64_t)nb * rs + lane * 8;

    f32x16 acc = zero16();
    const bool live = (lane & 31) < a.T;               // lanes of tokens < T
    for (int kb = w * SK_U; kb < kb_total; kb += SKD_NW * SK_U) {
        bf16x8 wv[SK_U], hv[SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int q = kb + u;                       // records and H are in ring order
            const int k = q / kbF, lk = q - k * kbF;
            wv[u] = load_weight_frag(base + (int64_t)k * a.shard_elems + (int64_t)lk * 512);
            hv[u] = live ? load_frag(a.h + (int64_t)q * 512 + lane * 8)   // fragment-ordered H
                         : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
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
    // whole hidden-group pairs per shard; every wave gets the same number of
    // SK_U-block pieces
    const int64_t kb_gu = d / 16, kb_dn = (int64_t)P * (F / 16);
    return d % 64 == 0 && F % (32 * SK_G) == 0 && kb_gu % (SKG_NW * SK_U) == 0 &&
           kb_dn % (SKD_NW * SK_U) == 0;
}

hipError_t launch_gateup_skinny(const Bf16Args& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.P * (a.F / (32 * SK_G))));
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
