// Skinny-T (T <= 48) weight-streaming kernels of the sharded MLP (gfx950).
//
// With few tokens every weight byte is used for few tokens, so the block is
// bound by reading the packed weights from HBM once. The packed 32 x 16
// fragment blocks are contiguous 1 KiB pieces, so each wave load is a fully
// coalesced 16 bytes per lane; the tokens come from L2 as NTB blocks of 32
// MFMA columns (NTB = 1 for T <= 32, 2 for T <= 48; columns past T are zero).
// The MFMA is v_mfma_f32_32x32x16_bf16.
//
// skinny_gateup: one workgroup per G groups of 32 hidden columns of one shard
//   (records and the hidden columns they produce are both stored in ring
//   order), so each token fragment it loads feeds 2 G (SwiGLU) or G weight
//   blocks. Its waves take the model dimension's fragment blocks in an
//   interleaved order (wave w: blocks w * SK_U + i * NW * SK_U ..), so the
//   workgroup reads each weight row front to back as one stream. Each wave
//   keeps fp32 accumulators; per token block the partial sums are added in
//   LDS in wave order, and wave g applies the activation for group g and
//   writes the 32 hidden bf16 values of every token straight into the MFMA
//   token-fragment order the down product reads (see below).
// skinny_down: one workgroup per 32 output features. The reduction runs over
//   all shards in ring order, flattened to one range of fragment blocks that
//   the waves take interleaved like the gate/up kernel; the per-wave partial
//   sums are added in wave order (a fixed order, so results are bitwise
//   reproducible) and the fp32 result goes straight to Y.
//
// Skinny hidden-activation layout (library workspace): for token block tb and
// every 16 hidden indices (ring-step order) one 1 KiB fragment block, at block
// tb * f / 16 + index / 16; lane l holds token 32 tb + l % 32 and hidden
// indices 8 (l / 32) .. + 7, so the down product loads its token operand with
// one contiguous 16-byte-per-lane access, like a weight block. Slots of tokens
// >= T are never written nor read (those lanes feed a zero operand instead).
//
// Measured on the 70B decode shape: two token blocks beat the tiled kernels
// up to T = 48 (255 vs 285 us at T = 33); at T = 64 the tokens' L2 traffic
// (two H fragments per weight fragment in the down product) makes them slower.
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

// NTB token blocks of 32 (T <= 32 NTB); G hidden groups and NW waves per
// workgroup (gate/up), NWD waves per workgroup (down).
template <int ACT, int NTB, int G, int NW>
__global__ __launch_bounds__(NW * 64) void skinny_gateup(Bf16Args a) {
    constexpr int NACC = ACT == 1 ? 2 : 1;
    constexpr int NR = G * NACC;
    __shared__ f32x16 red[NW][NR][1][64];
    poison_lds(red, sizeof(red));
    const int wg_per_shard = (a.F >> 5) / G;
    const int s = blockIdx.x / wg_per_shard;
    const int grp0 = (blockIdx.x - s * wg_per_shard) * G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kb_total = a.d >> 4;
    const int64_t rs = (int64_t)kb_total * 512;
    const uint16_t* p0 = a.packed + (int64_t)s * a.shard_elems + (int64_t)(grp0 * NACC) * rs + lane * 8;
    f32x16 acc[NR][NTB];
#pragma unroll
    for (int c = 0; c < NR; ++c)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) acc[c][tb] = zero16();
    for (int kb = w * SK_U; kb < kb_total; kb += NW * SK_U) {
        bf16x8 wv[NR][SK_U], xv[NTB][SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
#pragma unroll
            for (int c = 0; c < NR; ++c) wv[c][u] = load_weight_frag(p0 + c * rs + (int64_t)(kb + u) * 512);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
                xv[tb][u] = token_frag(a.x + (int64_t)tb * 32 * a.d, a.d, (int64_t)(kb + u) * 16, lane, a.T - tb * 32);
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u)
#pragma unroll
            for (int c = 0; c < NR; ++c)
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb)
                    acc[c][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[c][u], xv[tb][u], acc[c][tb], 0, 0, 0);
    }
    // token blocks are reduced one at a time through the same LDS buffer
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        if (tb > 0) __syncthreads();                    // the previous block's reads are done
#pragma unroll
        for (int c = 0; c < NR; ++c) red[w][c][0][lane] = acc[c][tb];
        __syncthreads();
        for (int g = w; g < G; g += NW) {
            const int grp = grp0 + g;
            f32x16 gs = red[0][g * NACC][0][lane], us = red[0][g * NACC + NACC - 1][0][lane];
#pragma unroll
            for (int i = 1; i < NW; ++i) {
                gs += red[i][g * NACC][0][lane];
                if (NACC == 2) us += red[i][g * NACC + 1][0][lane];
            }
            const int tok = lane & 31, h = lane >> 5;
            if (tb * 32 + tok < a.T) {
                const int64_t kb_base = (int64_t)tb * (a.f >> 4) + (((int64_t)s * a.F + grp * 32) >> 4);
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
}

template <int NTB, int NWD>
__global__ __launch_bounds__(NWD * 64) void skinny_down(Bf16Args a) {
    __shared__ f32x16 red[NWD][NTB][64];
    poison_lds(red, sizeof(red));
    const int nb = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int kbF = a.F >> 4;
    const int kb_total = a.P * kbF;
    const int64_t rs = (int64_t)kbF * 512;
    const uint16_t* base = a.packed + a.down_off + (int64_t)nb * rs + lane * 8;
    f32x16 acc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[tb] = zero16();
    for (int kb = w * SK_U; kb < kb_total; kb += NWD * SK_U) {
        bf16x8 wv[SK_U], hv[NTB][SK_U];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int q = kb + u;
            const int k = q / kbF, lk = q - k * kbF;
            wv[u] = load_weight_frag(base + (int64_t)k * a.shard_elems + (int64_t)lk * 512);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
                hv[tb][u] = tb * 32 + (lane & 31) < a.T
                    ? load_frag(a.h + ((int64_t)tb * (a.f >> 4) + q) * 512 + lane * 8)
                    : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u)
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
                acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[u], hv[tb][u], acc[tb], 0, 0, 0);
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) red[w][tb][lane] = acc[tb];
    __syncthreads();
    for (int tb = w; tb < NTB; tb += NWD) {
        f32x16 y = red[0][tb][lane];
#pragma unroll
        for (int i = 1; i < NWD; ++i) y += red[i][tb][lane];
        const int tok = tb * 32 + (lane & 31);
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
    // SK_U-block pieces (the two-token-block down kernel's 8 waves divide the
    // 16-wave condition)
    const int64_t kb_gu = d / 16, kb_dn = (int64_t)P * (F / 16);
    return d % 64 == 0 && F % (32 * SK_G) == 0 && kb_gu % (SKG_NW * SK_U) == 0 &&
           kb_dn % (SKD_NW * SK_U) == 0;
}

hipError_t launch_gateup_skinny(const Bf16Args& a, hipStream_t st) {
    if (a.T > SKINNY_T_MAX) return hipErrorInvalidValue;
    if (a.T <= 32) {
        const dim3 grid((unsigned)(a.P * (a.F / (32 * SK_G))));
        if (a.swiglu) hipLaunchKernelGGL((skinny_gateup<1, 1, SK_G, SKG_NW>), grid, dim3(SKG_NW * 64), 0, st, a);
        else hipLaunchKernelGGL((skinny_gateup<2, 1, SK_G, SKG_NW>), grid, dim3(SKG_NW * 64), 0, st, a);
    } else {
        const dim3 grid((unsigned)(a.P * (a.F / (32 * SK_G))));
        if (a.swiglu) hipLaunchKernelGGL((skinny_gateup<1, 2, SK_G, SKG_NW>), grid, dim3(SKG_NW * 64), 0, st, a);
        else hipLaunchKernelGGL((skinny_gateup<2, 2, SK_G, SKG_NW>), grid, dim3(SKG_NW * 64), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_down_skinny(const Bf16Args& a, hipStream_t st) {
    if (a.T > SKINNY_T_MAX) return hipErrorInvalidValue;
    if (a.T <= 32) hipLaunchKernelGGL((skinny_down<1, SKD_NW>), dim3((unsigned)(a.d / 32)), dim3(SKD_NW * 64), 0, st, a);
    else hipLaunchKernelGGL((skinny_down<2, 8>), dim3((unsigned)(a.d / 32)), dim3(8 * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace tsp
