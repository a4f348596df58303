// Backward pass of one rank's sharded gated MLP (gfx950).
//
// The gradients of the forward for an output gradient dY (the method's
// training step: "Folding Tensor and Sequence Parallelism ...", Abstract;
// "Tensor Parallelism: Splitting the Math", the paragraph after the
// walk-through names the backward pass beside the forward). For each shard s,
// visited in ring order like the forward:
//   dH_s = dY . Wd_s^T
//   SwiGLU: dG_s = dH_s * U_s * SiLU'(G_s), dU_s = dH_s * SiLU(G_s)
//   GeLU:   dU_s = dH_s * GeLU'(U_s)
//   dX  += dG_s . Wg_s^T + dU_s . Wu_s^T        (local accumulation, ring order)
//   dWg_s = X^T . dG_s, dWu_s = X^T . dU_s, dWd_s = H_s^T . dY   (the shard's own blocks)
// G_s, U_s and H_s are recomputed from X with the forward's gate/up kernel
// and packed records (gateup_bwd_w16), whose epilogue turns them into dG, dU
// and H. Every product runs on the shape-6 pipeline (w16.h); the backward's
// products read both operands row-major with the reduction index contiguous
// (RowSrc), so the token-reduced weight gradients read transposed copies of
// X, dY, dG, dU and H made by transpose_bf16 (padded with zero tokens to a
// multiple of 64).
#include "common.h"
#include "launch.h"
#include "w16.h"

namespace tsp {

// ------------------------------------------------------------------ transpose
// dst[c][r] = src[r][c] for r < R, 0 for R <= r < R_pad; 64 x 64 tiles through
// LDS, each thread moving 16 elements (two 16-byte accesses) each way.
__global__ __launch_bounds__(256) void transpose_bf16(const uint16_t* __restrict__ src, int R, int ld_src,
                                                      uint16_t* __restrict__ dst, int ld_dst) {
    __shared__ uint16_t tile[64][64 + 8];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
    const int r = r0 + tr;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (r < R) {
        const u32x4* p = reinterpret_cast<const u32x4*>(src + (int64_t)r * ld_src + c0 + tc);
        v0 = p[0];
        v1 = p[1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        tile[tr][tc + 2 * e] = (uint16_t)(v0[e] & 0xffffu);
        tile[tr][tc + 2 * e + 1] = (uint16_t)(v0[e] >> 16);
        tile[tr][tc + 8 + 2 * e] = (uint16_t)(v1[e] & 0xffffu);
        tile[tr][tc + 8 + 2 * e + 1] = (uint16_t)(v1[e] >> 16);
    }
    __syncthreads();
    // thread: output row c0 + tr, tokens r0 + tc .. + 15
    u32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o0[e] = (uint32_t)tile[tc + 2 * e][tr] | ((uint32_t)tile[tc + 2 * e + 1][tr] << 16);
        o1[e] = (uint32_t)tile[tc + 8 + 2 * e][tr] | ((uint32_t)tile[tc + 8 + 2 * e + 1][tr] << 16);
    }
    u32x4* q = reinterpret_cast<u32x4*>(dst + (int64_t)(c0 + tr) * ld_dst + r0 + tc);
    q[0] = o0;
    q[1] = o1;
}

// ------------------------------------------------------------------ NT product
// C[n][m] = sum_k A[m][k] B[n][k] on the shape-6 pipeline, fp32 out:
// out[row(n) * ldc + col(m)], n < N. remap 1: column m is a ring-ordered
// hidden index (ring step m / F) stored at its shard's natural column
// order[m / F] * F + m % F; remap 2: the same for the row n. F % 256 == 0, so
// a 256-wide tile never straddles two shards and the remap is one offset per
// tile.
//
// One launch runs up to three such products (NtGroup): workgroup ids are
// dealt out to the products in order, so products whose tile counts are not
// multiples of the CU count share one tail instead of leaving one each.
template <bool BUF>
__global__ __launch_bounds__(256) void nt_w16(NtGroup grp) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE];
    poison_lds(lds, sizeof(lds));
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int gi = lin < grp.first[1] ? 0 : (lin < grp.first[2] ? 1 : 2);
    const NtArgs& p = gi == 0 ? grp.p[0] : (gi == 1 ? grp.p[1] : grp.p[2]);
    const int n_mt = p.M / BM, n_nt = (p.N + BN - 1) / BN;
    int ntile, mtile;
    raster(lin - grp.first[gi], n_mt, n_nt, ntile, mtile);
    const int m0 = mtile * BM, n0 = ntile * BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    RowSrc<BUF> src;
    src.ls = 0;
    src.j = 0;
    src.spp = p.spp;
    src.nseg = p.nseg;
    src.kinds = p.kinds;
    src.a_base0 = p.a_base[0];
    src.a_base1 = p.a_base[1];
    src.b_base0 = p.b_base[0];
    src.b_base1 = p.b_base[1];
    src.a_seg = p.a_seg;
    src.b_seg = p.b_seg;
    src.order = p.order;
    src.lda = p.lda;
    src.ldb = p.ldb;
    src.m0 = m0;
    src.n0 = n0;
    src.last_m = p.M - 1;
    src.last_n = p.N - 1;
    src.w = __builtin_amdgcn_readfirstlane(w);
    src.wm = wm;
    src.wn = wn;
    src.lane = lane;
    src.seek(0);
    f32x4 acc[TM][TN];
    w16::mainloop(lds, acc, p.spp * p.nseg, src);

    int64_t col0 = m0, row_shift = 0;
    if (p.remap == 1) col0 = (int64_t)p.remap_order[m0 / p.F] * p.F + m0 % p.F;
    if (p.remap == 2) row_shift = (int64_t)p.remap_order[n0 / p.F] * p.F + n0 % p.F - n0;
    // Output rows are the N side, so a store straight from the MFMA layout
    // would write 16 rows x 64 bytes; the tile goes out through the LDS ring
    // instead, half of each wave row's tokens at a time, one 1 KiB row per store.
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
        stg.flush(p.out, p.ldc, n0, p.N, row_shift, col0, w, lane, hh);
        lgkm_zero();
    }
}

// ------------------------------------------------------------------ gate/up backward
// The forward's gate/up product (packed records in ring order, shape 6), with
// an epilogue that reads dH at the shard's natural hidden columns and writes
// dG, dU and H (bf16, ring-ordered hidden columns like the forward's H).
// SiLU'(g) = sigma (1 + g (1 - sigma)); with z2 = sqrt(8/pi) (u + 0.044715 u^3),
// GeLU(u) = u sigma2 and GeLU'(u) = sigma2 (1 + u (1 - sigma2) dz2/du), where
// sigma = 1 / (1 + e^-g) and sigma2 = 1 / (1 + e^-z2) (the tanh form,
// 1 + tanh(z2 / 2) = 2 sigma2). Reciprocals use v_rcp_f32 as in the forward.
__device__ inline float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

template <int ACT, bool BUF>
__global__ __launch_bounds__(256) void gateup_bwd_w16(Bf16Args a, BwdArgs b, int n_ft_shard, int n_tt) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE];
    poison_lds(lds, sizeof(lds));
    int ttile, flin;
    raster(xcd_remap(blockIdx.x, gridDim.x), a.P * n_ft_shard, n_tt, ttile, flin);
    const int k = flin / n_ft_shard;                    // ring step (record index)
    const int ftile = flin - k * n_ft_shard;
    const int64_t a_rs = (int64_t)(a.d >> 4) * 512;
    const uint16_t* a_tile = a.packed + (int64_t)k * a.shard_elems + (int64_t)(ftile * (BM / 32)) * a_rs;
    const int t0 = ttile * BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    PackedSrc<BUF> src{a_tile, 0, 0, a.d >> 5, 0, 0, a_rs, a.x, a.d, t0, a.T,
                       __builtin_amdgcn_readfirstlane(w), wm, wn, lane};
    f32x4 acc[TM][TN];
    w16::mainloop(lds, acc, a.d >> 5, src);

    // Epilogue. The tile covers hidden columns [lc0, lc0 + COLS) of shard
    // order[k] (COLS = 128 for SwiGLU, 256 for GeLU): dH is read at the shard's
    // natural columns, dG, dU and H are written at the ring-ordered columns.
    // All of them go through the LDS ring (StagedRows16) so that the stores
    // write whole rows, in two halves of the tokens: a half of all outputs
    // fits in the ring, and the accumulators a half consumes die with it.
    constexpr int COLS = ACT == 1 ? BM / 2 : BM;
    constexpr int NB = ACT == 1 ? 4 : TM;               // 16-column blocks of the wave
    constexpr int NO = ACT == 1 ? 3 : 2;                // outputs
    using Stg = StagedRows16<COLS, 128>;
    static_assert(NO * Stg::ELEMS <= NS * STAGE, "LDS");
    const int lc0 = ftile * COLS;
    const int64_t ring0 = (int64_t)k * a.F + lc0, nat0 = (int64_t)b.order[k] * a.F + lc0;
    const int fsub = 4 * (lane >> 4);
    const float* __restrict__ dh = b.dh;
    Stg sh{lds}, su{lds + Stg::ELEMS}, sg_{lds + 2 * Stg::ELEMS};
    auto col = [&](int ib) { return ACT == 1 ? (wm * 2 + ib / 2) * 32 + (ib % 2) * 16 + fsub
                                             : (wm * TM + ib) * 16 + fsub; };
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        stage_barrier();                                // fragment reads / the last flush's reads are done
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
            const int c = col(ib);
            // the dH values of the half's four (16-token, 4-column) pieces are
            // loaded together before any of them is used
            f32x4 dv[TN / 2];
#pragma unroll
            for (int jj = 0; jj < TN / 2; ++jj) {
                const int tok = min(t0 + wn * 128 + hh * 64 + jj * 16 + (lane & 15), a.T - 1);
                dv[jj] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4*>(dh + (int64_t)tok * a.f + nat0 + c));
            }
#pragma unroll
            for (int jj = 0; jj < TN / 2; ++jj) {
                const int j = hh * (TN / 2) + jj, r = wn * 64 + jj * 16 + (lane & 15);
                if constexpr (ACT == 1) {
                    // wave rows: 16-row blocks 4 q + i gate and 4 q + 2 + i up
                    // of hidden group q = ib / 2, i = ib % 2 (see the forward)
                    const f32x4 g = acc[4 * (ib / 2) + ib % 2][j], u = acc[4 * (ib / 2) + 2 + ib % 2][j];
                    float dg[4], du[4], h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float sg = sigmoid_f(g[e]);
                        const float si = g[e] * sg;
                        dg[e] = dv[jj][e] * u[e] * (sg * (1.0f + g[e] * (1.0f - sg)));
                        du[e] = dv[jj][e] * si;
                        h[e] = si * u[e];
                    }
                    sg_.put4(r, c, pack4_bf16(dg[0], dg[1], dg[2], dg[3]));
                    su.put4(r, c, pack4_bf16(du[0], du[1], du[2], du[3]));
                    sh.put4(r, c, pack4_bf16(h[0], h[1], h[2], h[3]));
                } else {
                    const f32x4 u = acc[ib][j];
                    float du[4], h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = u[e];
                        const float z2 = 1.5957691216057308f * (x + 0.044715f * x * x * x);
                        const float dz2 = 1.5957691216057308f * (1.0f + 3.0f * 0.044715f * x * x);
                        const float s2 = sigmoid_f(z2);
                        du[e] = dv[jj][e] * (s2 * (1.0f + x * (1.0f - s2) * dz2));
                        h[e] = x * s2;
                    }
                    su.put4(r, c, pack4_bf16(du[0], du[1], du[2], du[3]));
                    sh.put4(r, c, pack4_bf16(h[0], h[1], h[2], h[3]));
                }
            }
        }
        lgkm_zero();
        stage_barrier();
        if constexpr (ACT == 1) sg_.flush(b.dg, a.f, t0, a.T, ring0, w, lane, hh);
        su.flush(b.du, a.f, t0, a.T, ring0, w, lane, hh);
        sh.flush(b.h, a.f, t0, a.T, ring0, w, lane, hh);
        lgkm_zero();
    }
}

// ------------------------------------------------------------------ launchers
static inline int64_t cdiv64(int64_t x, int64_t y) { return (x + y - 1) / y; }

hipError_t launch_transpose_bf16(const uint16_t* src, int R, int C, int ld_src, uint16_t* dst, int R_pad,
                                 hipStream_t st) {
    if (C % 64 || R_pad % 64 || R > R_pad) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)(C / 64), (unsigned)(R_pad / 64)), dim3(256), 0, st, src, R,
                       ld_src, dst, R_pad);
    return hipGetLastError();
}

hipError_t launch_nt(const NtArgs* probs, int n, hipStream_t st) {
    using namespace w16;
    if (n < 1 || n > 3) return hipErrorInvalidValue;
    NtGroup grp{};
    int64_t tiles = 0;
    // buffer offsets are 32-bit: every row of either operand must lie within
    // 2^31 bytes of that operand's base
    bool buf = true;
    for (int i = 0; i < 3; ++i) {
        grp.first[i] = (int)tiles;
        if (i >= n) continue;
        const NtArgs& p = probs[i];
        if (p.M % BM || p.N < 1 || (p.spp * p.nseg) % 2 || p.spp * p.nseg < 2 || p.kinds < 1 || p.kinds > 2)
            return hipErrorInvalidValue;
        if (p.remap && (p.F % BM || !p.remap_order)) return hipErrorInvalidValue;
        grp.p[i] = p;
        tiles += (int64_t)(p.M / BM) * cdiv64(p.N, BN);
        buf = buf && (int64_t)p.M * p.lda * 2 < (int64_t(1) << 31) && (int64_t)p.N * p.ldb * 2 < (int64_t(1) << 31);
    }
    for (int i = n; i < 3; ++i) grp.first[i] = (int)tiles;
    if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles);
    if (buf) hipLaunchKernelGGL((nt_w16<true>), grid, dim3(256), 0, st, grp);
    else hipLaunchKernelGGL((nt_w16<false>), grid, dim3(256), 0, st, grp);
    return hipGetLastError();
}

hipError_t launch_gateup_bwd(const Bf16Args& a, const BwdArgs& b, hipStream_t st) {
    const int ngu = a.swiglu ? 2 * a.F : a.F;
    if (ngu % 256 || a.d % 64) return hipErrorInvalidValue;
    const int n_ft_shard = ngu / 256, n_tt = (int)cdiv64(a.T, 256);
    const dim3 grid((unsigned)(a.P * n_ft_shard * n_tt));
    const bool buf = (int64_t)a.T * a.d * 2 < (int64_t(1) << 31) && (int64_t)a.d * 512 < (int64_t(1) << 31);
    if (a.swiglu) {
        if (buf) hipLaunchKernelGGL((gateup_bwd_w16<1, true>), grid, dim3(256), 0, st, a, b, n_ft_shard, n_tt);
        else hipLaunchKernelGGL((gateup_bwd_w16<1, false>), grid, dim3(256), 0, st, a, b, n_ft_shard, n_tt);
    } else {
        if (buf) hipLaunchKernelGGL((gateup_bwd_w16<2, true>), grid, dim3(256), 0, st, a, b, n_ft_shard, n_tt);
        else hipLaunchKernelGGL((gateup_bwd_w16<2, false>), grid, dim3(256), 0, st, a, b, n_ft_shard, n_tt);
    }
    return hipGetLastError();
}

}  // namespace tsp
