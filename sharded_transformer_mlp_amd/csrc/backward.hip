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
// and H. Every product runs on the 256 x 256 pipeline (w16.h) with both
// operands' reduction index contiguous (RowSrc): the B operand row-major, the
// A operand row-major (dH: Wd) or in 32 x 16 fragment blocks (dX: Wg, Wu
// packed once from the records; the weight gradients: dG^T, dU^T written so
// by the gate/up epilogue, dY^T by the transposes of the dH launch). The token-reduced weight
// gradients read transposed copies of X, dY, dG, dU and H (tokens padded with
// zeros, or finite values facing zeros, to a multiple of 64).
#include "common.h"
#include "launch.h"
#include "w16.h"

namespace tsp {

// ------------------------------------------------------------------ transpose
// dst[c][r] = src[r][c] for r < R, 0 for R <= r < R_pad; 64 x 64 tiles through
// LDS, each thread moving 16 elements (two 16-byte accesses) each way. frag:
// dst in 32 x 16 fragment blocks (rows c, reduction index r, ld_dst / 16
// blocks per 32-row block), where a thread's two 8-token runs are the two
// 16-byte lane slots (l, l + 32) of one block. The tiles run as extra
// workgroups of a grouped NT launch (tp_aux), so that they fill the CUs the
// product's last partial round leaves idle instead of taking a launch of
// their own.
typedef uint16_t TpTile[64][64 + 2];                // 33-word rows: the column reads spread over the banks

// Tile (cb, rb) of job j: thread's 16 source elements into v[0..1] (zeros past R).
__device__ __forceinline__ void tp_load(const TransposeJob& j, int cb, int rb, u32x4 (&v)[2]) {
    const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
    const int r = rb * 64 + tr;
    v[0] = u32x4{0u, 0u, 0u, 0u};
    v[1] = u32x4{0u, 0u, 0u, 0u};
    if (r < j.R) {
        const u32x4* p = reinterpret_cast<const u32x4*>(j.src + (int64_t)r * j.ld_src + cb * 64 + tc);
        v[0] = p[0];
        v[1] = p[1];
    }
}
__device__ __forceinline__ void tp_put(TpTile& tile, const u32x4 (&v)[2]) {
    const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        tile[tr][tc + 2 * e] = (uint16_t)(v[0][e] & 0xffffu);
        tile[tr][tc + 2 * e + 1] = (uint16_t)(v[0][e] >> 16);
        tile[tr][tc + 8 + 2 * e] = (uint16_t)(v[1][e] & 0xffffu);
        tile[tr][tc + 8 + 2 * e + 1] = (uint16_t)(v[1][e] >> 16);
    }
}
// after tp_put of the whole tile and a barrier: thread writes output row
// c0 + tr, tokens r0 + tc .. + 15
__device__ __forceinline__ void tp_store(const TpTile& tile, const TransposeJob& j, int cb, int rb) {
    const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
    const int c0 = cb * 64, r0 = rb * 64;
    u32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o0[e] = (uint32_t)tile[tc + 2 * e][tr] | ((uint32_t)tile[tc + 2 * e + 1][tr] << 16);
        o1[e] = (uint32_t)tile[tc + 8 + 2 * e][tr] | ((uint32_t)tile[tc + 8 + 2 * e + 1][tr] << 16);
    }
    const int64_t row = c0 + tr;
    if (j.frag) {
        u32x4* q = reinterpret_cast<u32x4*>(j.dst + ((row >> 5) * (j.R_pad >> 4) + ((r0 + tc) >> 4)) * 512 +
                                            (row & 31) * 8);
        q[0] = o0;                                      // lane slot row % 32: tokens r0 + tc .. + 7
        q[32] = o1;                                     // lane slot row % 32 + 32: the next 8
    } else {
        u32x4* q = reinterpret_cast<u32x4*>(j.dst + row * j.R_pad + r0 + tc);
        q[0] = o0;
        q[1] = o1;
    }
}

// Aux workgroup `id` of n_aux: tiles id, id + n_aux, ... of the jobs' tiles
// taken in order (job 0's C/64 x R_pad/64, then job 1's). TP_DEPTH tiles'
// loads are in flight at a time; the LDS tile alternates between two
// buffers, so one barrier per tile separates a buffer's writes from its reads
// and (two tiles on) its reads from its next writes. The trip count depends
// on id and the sizes only: every wave of the workgroup reaches every barrier.
constexpr int TP_DEPTH = 4;
__device__ __forceinline__ void tp_aux(const TransposeJob j0, const TransposeJob j1, int n_tp, int n_aux, int id,
                                       uint16_t* lds) {
    TpTile* tiles = reinterpret_cast<TpTile*>(lds);
    const int n0 = (j0.C / 64) * (j0.R_pad / 64);
    const int total = n0 + (n_tp > 1 ? (j1.C / 64) * (j1.R_pad / 64) : 0);
    // tile t: job, column block cb, row block rb
    auto locate = [&](int t, int& job, int& cb, int& rb) {
        job = t < n0 ? 0 : 1;
        const int u = t < n0 ? t : t - n0;
        const int ncb = (job ? j1.C : j0.C) / 64;
        rb = u / ncb;
        cb = u - rb * ncb;
    };
    auto load = [&](int t, u32x4 (&v)[2]) {
        int job, cb, rb;
        locate(t, job, cb, rb);
        tp_load(job ? j1 : j0, cb, rb, v);
    };
    u32x4 v[TP_DEPTH][2];
#pragma unroll
    for (int k = 0; k < TP_DEPTH; ++k)
        if (id + k * n_aux < total) load(id + k * n_aux, v[k]);
    for (int base = id; base < total; base += TP_DEPTH * n_aux) {
#pragma unroll
        for (int k = 0; k < TP_DEPTH; ++k) {
            const int t = base + k * n_aux;
            if (t < total) {                            // uniform over the workgroup
                int job, cb, rb;
                locate(t, job, cb, rb);
                tp_put(tiles[k & 1], v[k]);
                __syncthreads();
                tp_store(tiles[k & 1], job ? j1 : j0, cb, rb);
                if (t + TP_DEPTH * n_aux < total) load(t + TP_DEPTH * n_aux, v[k]);
            }
        }
    }
}

// ------------------------------------------------------------------ NT product
// C[n][m] = sum_k A[m][k] B[n][k] on the 256 x 256 pipeline, fp32 out:
// out[row(n) * ldc + col(m)], n < N. remap 1: column m is a ring-ordered
// hidden index (ring step m / F) stored at its shard's natural column
// order[m / F] * F + m % F; remap 2: the same for the row n. F % 256 == 0, so
// a 256-wide tile never straddles two shards and the remap is one offset per
// tile.
//
// One launch runs up to four such products (NtGroup): workgroup ids are
// dealt out to the products in order, so products whose tile counts are not
// multiples of the CU count share one tail instead of leaving one each (the
// backward puts its long-reduction dX tiles last, where they start on the CUs
// that the weight gradients' last partial round leaves idle). Each product's
// range of workgroup ids starts at a multiple of 8 and is remapped to XCDs on
// its own, so every product's tiles spread over all eight XCDs (remapped as one
// range, the last product's tiles would all land on the last XCD).
template <bool BUF, bool FRAG>
__global__ __launch_bounds__(256) void nt_w16(NtGroup grp) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
    poison_lds(lds, sizeof(lds));
    const int bid = blockIdx.x;
    if (bid >= grp.aux_first) {                         // a transpose workgroup (launch_nt's tps)
        tp_aux(grp.tp[0], grp.tp[1], grp.n_tp, grp.n_aux, bid - grp.aux_first, lds);
        return;
    }
    const int gi = bid < grp.first[1] ? 0 : (bid < grp.first[2] ? 1 : (bid < grp.first[3] ? 2 : 3));
    const NtArgs& p = gi == 0 ? grp.p[0] : (gi == 1 ? grp.p[1] : (gi == 2 ? grp.p[2] : grp.p[3]));
    const int n_mt = p.M / BM, n_nt = (p.N + BN - 1) / BN;
    const int first = gi == 0 ? grp.first[0] : (gi == 1 ? grp.first[1] : (gi == 2 ? grp.first[2] : grp.first[3]));
    const int next = gi == 0 ? grp.first[1] : (gi == 1 ? grp.first[2] : (gi == 2 ? grp.first[3] : grp.aux_first));
    const int lin = xcd_remap(bid - first, next - first);
    if (lin >= n_mt * n_nt) return;                     // padding of the product's id range to a multiple of 8
    int ntile, mtile;
    raster(lin, n_mt, n_nt, ntile, mtile);
    const int m0 = mtile * BM, n0 = ntile * BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    RowSrc<BUF, FRAG> src;
    src.ls = 0;
    src.j = 0;
    src.lsb = 0;
    src.jb = 0;
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
    src.seek_a(0);
    src.seek_b(0);
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
// The forward's gate/up product (packed records in ring order, tile shape 0), with
// an epilogue that reads dH at the shard's natural hidden columns and writes
// dG, dU and H (bf16, ring-ordered hidden columns like the forward's H).
// SiLU'(g) = sigma (1 + g (1 - sigma)); with z2 = sqrt(8/pi) (u + 0.044715 u^3),
// GeLU(u) = u sigma2 and GeLU'(u) = sigma2 (1 + u (1 - sigma2) dz2/du), where
// sigma = 1 / (1 + e^-g) and sigma2 = 1 / (1 + e^-z2) (the tanh form,
// 1 + tanh(z2 / 2) = 2 sigma2). Reciprocals use v_rcp_f32 as in the forward.
__device__ inline float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// SAVED: the accumulators come from a forward's saved pre-activations
// (b.saved, w16::save_acc's layout, bit for bit what the product would give)
// instead of the product, and the epilogue is the same.
template <int ACT, bool BUF, bool SAVED>
__global__ __launch_bounds__(256) void gateup_bwd_w16(Bf16Args a, BwdArgs b, int n_ft_shard, int n_tt) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
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
    if constexpr (SAVED) load_acc(b.saved, (int64_t)flin * n_tt + ttile, __builtin_amdgcn_readfirstlane(w), lane, acc);
    else w16::mainloop(lds, acc, a.d >> 5, src);

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
    static_assert(NO * Stg::ELEMS <= LDS_ELEMS, "LDS");
    const int lc0 = ftile * COLS;
    const int64_t ring0 = (int64_t)k * a.F + lc0, nat0 = (int64_t)b.order[k] * a.F + lc0;
    const int fsub = 4 * (lane >> 4);
    const float* __restrict__ dh = b.dh;
    Stg sh{lds}, su{lds + Stg::ELEMS}, sg_{lds + 2 * Stg::ELEMS};
    auto col = [&](int ib) { return ACT == 1 ? (wm * 2 + ib / 2) * 32 + (ib % 2) * 16 + fsub
                                             : (wm * TM + ib) * 16 + fsub; };
    // dH of (half hh, block ib): the half's four (16-token, 4-column) pieces
    // of the lane, loaded one block ahead of their use (two blocks' worth of
    // registers), so that a block's arithmetic covers the next block's loads
    auto load_dh = [&](int hh, int ib, f32x4 (&dv)[TN / 2]) {
        const int c = col(ib);
#pragma unroll
        for (int jj = 0; jj < TN / 2; ++jj) {
            const int tok = min(t0 + wn * 128 + hh * 64 + jj * 16 + (lane & 15), a.T - 1);
            dv[jj] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dh + (int64_t)tok * a.f + nat0 + c));
        }
    };
    f32x4 dvb[2][TN / 2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        load_dh(hh, 0, dvb[0]);
        stage_barrier();                                // fragment reads / the last flush's reads are done
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
            const int c = col(ib);
            if (ib + 1 < NB) load_dh(hh, ib + 1, dvb[(ib + 1) & 1]);
            const f32x4 (&dv)[TN / 2] = dvb[ib & 1];
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
            // at most two blocks' dH loads in flight: hoisting every block's
            // loads ahead of the arithmetic (8 blocks x 16 registers for GeLU)
            // ran the kernel out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
        lgkm_zero();
        stage_barrier();
        // dG and dU row-major for dX, and transposed (tokens contiguous) for
        // the weight gradients, which reduce over tokens: dG, dU as their A
        // operands (fragment blocks), H as a B operand (row-major)
        if constexpr (ACT == 1) {
            sg_.flush(b.dg, a.f, t0, a.T, ring0, w, lane, hh);
            flush_frag_transposed(sg_, b.dgt, b.ldt, ring0, t0, hh, (int)threadIdx.x);
        }
        su.flush(b.du, a.f, t0, a.T, ring0, w, lane, hh);
        flush_frag_transposed(su, b.dut, b.ldt, ring0, t0, hh, (int)threadIdx.x);
        flush_transposed(sh, b.ht, b.ldt, ring0, t0, hh, (int)threadIdx.x);
        lgkm_zero();
    }
}

// ------------------------------------------------------------------ launchers
static inline int64_t cdiv64(int64_t x, int64_t y) { return (x + y - 1) / y; }

hipError_t launch_nt(const NtArgs* probs, int n, hipStream_t st, const TransposeJob* tps, int n_tp) {
    using namespace w16;
    if (n < 1 || n > kMaxNt) return hipErrorInvalidValue;
    NtGroup grp{};
    int64_t tiles = 0;
    // buffer offsets are 32-bit: every row of either operand must lie within
    // 2^31 bytes of that operand's base
    bool buf = true;
    for (int i = 0; i < kMaxNt; ++i) {
        grp.first[i] = (int)tiles;                      // a multiple of 8 (see nt_w16)
        if (i >= n) continue;
        const NtArgs& p = probs[i];
        if (p.M % BM || p.N < 1 || (p.spp * p.nseg) % 2 || p.spp * p.nseg < 2 || p.kinds < 1 || p.kinds > 2)
            return hipErrorInvalidValue;
        if (p.remap && (p.F % BM || !p.remap_order)) return hipErrorInvalidValue;
        // fragment-block A: every segment's reduction range lies inside the K = lda indices
        if (p.a_frag != probs[0].a_frag ||
            (p.a_frag && (p.lda % 32 || p.nseg % p.kinds ||
                          (int64_t)(p.nseg / p.kinds - 1) * p.a_seg + (int64_t)p.spp * 32 > p.lda)))
            return hipErrorInvalidValue;
        grp.p[i] = p;
        tiles += cdiv64((int64_t)(p.M / BM) * cdiv64(p.N, BN), 8) * 8;
        buf = buf && (int64_t)p.M * p.lda * 2 < (int64_t(1) << 31) && (int64_t)p.N * p.ldb * 2 < (int64_t(1) << 31);
    }
    for (int i = n; i < kMaxNt; ++i) grp.first[i] = (int)tiles;
    if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
    // transposes: as many workgroups as the products' last round leaves CUs
    // idle (a full round's worth when that is under 64)
    if (n_tp < 0 || n_tp > kMaxTp || (n_tp > 0 && !tps)) return hipErrorInvalidValue;
    grp.n_tp = n_tp;
    grp.aux_first = (int)tiles;
    grp.n_aux = 0;
    if (n_tp > 0) {
        int64_t tp_tiles = 0;
        for (int i = 0; i < n_tp; ++i) {
            const TransposeJob& j = tps[i];
            if (!j.src || !j.dst || j.R < 0 || j.C < 64 || j.C % 64 || j.R_pad % 64 || j.R > j.R_pad || j.R_pad < 64 ||
                j.ld_src < j.C || j.ld_src % 8)
                return hipErrorInvalidValue;
            grp.tp[i] = j;
            tp_tiles += (int64_t)(j.C / 64) * (j.R_pad / 64);
        }
        if (tp_tiles > INT32_MAX / 2) return hipErrorInvalidValue;
        int dev = 0, n_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        n_cu = std::max(n_cu, 1);
        const int idle = (int)((n_cu - tiles % n_cu) % n_cu);
        grp.n_aux = (int)std::min<int64_t>(idle >= 64 ? idle : n_cu, tp_tiles);
        tiles += grp.n_aux;
    }
    const dim3 grid((unsigned)tiles);
    if (probs[0].a_frag) {
        if (buf) hipLaunchKernelGGL((nt_w16<true, true>), grid, dim3(256), 0, st, grp);
        else hipLaunchKernelGGL((nt_w16<false, true>), grid, dim3(256), 0, st, grp);
    } else {
        if (buf) hipLaunchKernelGGL((nt_w16<true, false>), grid, dim3(256), 0, st, grp);
        else hipLaunchKernelGGL((nt_w16<false, false>), grid, dim3(256), 0, st, grp);
    }
    return hipGetLastError();
}

hipError_t launch_gateup_bwd(const Bf16Args& a, const BwdArgs& b, hipStream_t st) {
    const int ngu = a.swiglu ? 2 * a.F : a.F;
    if (ngu % 256 || a.d % 64) return hipErrorInvalidValue;
    const int n_ft_shard = ngu / 256, n_tt = (int)cdiv64(a.T, 256);
    const dim3 grid((unsigned)(a.P * n_ft_shard * n_tt));
    const bool buf = (int64_t)a.T * a.d * 2 < (int64_t(1) << 31) && (int64_t)a.d * 512 < (int64_t(1) << 31);
#define TSP_GB(ACT, BUF, SAVED) hipLaunchKernelGGL((gateup_bwd_w16<ACT, BUF, SAVED>), grid, dim3(256), 0, st, a, b, n_ft_shard, n_tt)
    if (a.swiglu) {
        if (b.saved) TSP_GB(1, true, true);
        else if (buf) TSP_GB(1, true, false);
        else TSP_GB(1, false, false);
    } else {
        if (b.saved) TSP_GB(2, true, true);
        else if (buf) TSP_GB(2, true, false);
        else TSP_GB(2, false, false);
    }
#undef TSP_GB
    return hipGetLastError();
}

int64_t gateup_saved_bytes(int64_t T, int64_t F, int P, int swiglu) {
    const int64_t n_ft_shard = (swiglu ? 2 * F : F) / 256, n_tt = cdiv64(T, 256);
    return (int64_t)P * n_ft_shard * n_tt * w16::BM * w16::BN * 4;
}

}  // namespace tsp
