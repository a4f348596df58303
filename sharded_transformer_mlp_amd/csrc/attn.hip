// One rank's attention block under TSP on gfx950: the head-group shards in
// the rank's visiting order, each projected (Q, K, V columns of the group),
// its keys and values placed in the sequence-wide context, causal softmax
// attention of the rank's queries over that context, and the group's output
// projection added into the rank's fp32 output.
//
// "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
// Training & Inference", Abstract: for attention the ranks go through the
// broadcast parameter shards one after another and rebuild the context with a
// sequence-wise key/value exchange. "Tensor Parallelism: Splitting the Math",
// section "Why the column-then-row split - and what happens in attention":
// Q, K, V projections split by heads (columns), the output projection by the
// matching rows. On one GPU the exchange is the context buffer: each rank's
// projection writes its own rows of it (positions [rank T, (rank + 1) T)).
//
// Kernels:
//   pack_qkv_bf16  packs head group s's columns of Wq, Wk, Wv as one record
//                  (Q heads, then K heads, then V heads), in the MLP's
//                  fragment-block layout, records in visiting order.
//   qkv_w16        the projection: the MLP's 256 x 256 pipeline (w16.h) over
//                  the records with a plain epilogue that rounds to fp16 and
//                  sends each 128-column head to its place: Q to the rank's
//                  query buffer, K rows to the key context, V transposed to
//                  the value context.
//   attn_fwd       (attn_core.hip) the attention itself; the output
//                  projection is the MLP's down product (gemm_tiled.hip).
#include "attn.h"
#include "common.h"
#include "launch.h"
#include "w16.h"

namespace tsp {

// ------------------------------------------------------------------ packing

// Record k (head group s = order[k]) holds Fqkv = (Hs + 2 Hks) dh packed
// features: feature j < Hs dh is column s Hs dh + j of Wq, the next Hks dh are
// columns of Wk from s Hks dh, the last Hks dh the same columns of Wv. Same
// fragment-block order as the MLP's gate/up part (common.h).
__global__ void pack_qkv_bf16(const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
                              const uint16_t* __restrict__ wv, uint16_t* __restrict__ dst,
                              const int32_t* __restrict__ order, int64_t rec_elems, int d, int ldq, int ldkv,
                              int Fq, int Fk, int64_t chunks) {
    const int rec = blockIdx.y;
    const int s = order[rec];
    const int kblocks = d >> 4;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = c >> 6;
        const int lane = (int)(c & 63);
        const int64_t nb = block / kblocks;
        const int kb = (int)(block - nb * kblocks);
        const int64_t j = nb * 32 + (lane & 31);
        const int k0 = kb * 16 + (lane >> 5) * 8;
        const uint16_t* src;
        int64_t col, ld;
        if (j < Fq) {
            src = wq; col = (int64_t)s * Fq + j; ld = ldq;
        } else if (j < Fq + Fk) {
            src = wk; col = (int64_t)s * Fk + (j - Fq); ld = ldkv;
        } else {
            src = wv; col = (int64_t)s * Fk + (j - Fq - Fk); ld = ldkv;
        }
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[(int64_t)(k0 + e) * ld + col];
        u32x4 o = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                   v[6] | ((uint32_t)v[7] << 16)};
        *reinterpret_cast<u32x4*>(dst + (int64_t)rec * rec_elems + c * 8) = o;
    }
}

// ------------------------------------------------------------------ projection

template <bool BUF>
__global__ __launch_bounds__(256) void qkv_w16(ProjArgs a, int n_ft_shard, int n_tt) {
    using namespace w16;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
    poison_lds(lds, sizeof(lds));
    int ttile, flin;
    raster(xcd_remap(blockIdx.x, gridDim.x), a.P * n_ft_shard, n_tt, ttile, flin);
    const int k = flin / n_ft_shard;
    const int ftile = flin - k * n_ft_shard;
    const int64_t a_rs = (int64_t)(a.d >> 4) * 512;
    const uint16_t* a_tile = a.packed + (int64_t)k * a.rec_elems + (int64_t)(ftile * (BM / 32)) * a_rs;
    const int t0 = ttile * BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    PackedSrc<BUF> src{a_tile, 0, 0, a.d >> 5, 0, 0, a_rs, a.x, a.d, t0, a.T,
                       __builtin_amdgcn_readfirstlane(w), wm, wn, lane};
    f32x4 acc[TM][TN];
    w16::mainloop(lds, acc, a.d >> 5, src);

    // the tile (256 tokens x 256 features) through the LDS ring, then each
    // 128-feature half, one head, to its destination. Query heads are scaled
    // by q_scale (the softmax's log2(e)/sqrt(dh)) before their one rounding,
    // so that the attention's scores come out in log2 units.
    StagedRows16<BM> stg{lds};
    stage_barrier();
    const int fsub = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int c = (wm * TM + i) * 16 + fsub;
        const float sc = ftile * 2 + (c >> 7) < a.Hs ? a.q_scale : 1.0f;   // head slot of column c
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const f32x4 u = acc[i][j] * sc;
            stg.put4((wn * TN + j) * 16 + (lane & 15), c, pack4_f16(u[0], u[1], u[2], u[3]));
        }
    }
    lgkm_zero();
    stage_barrier();
    const int s = a.order[k];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int slot = ftile * 2 + hf;                // head slot in the record: Q heads, K heads, V heads
        const int c0 = hf * 128;
        if (slot < a.Hs + a.Hks) {
            // rows: Q to the query buffer (ring-ordered groups), K to the key
            // context at the tokens' sequence positions
            uint16_t* dst;
            int64_t ld, r0;
            if (slot < a.Hs) {
                dst = a.q + ((int64_t)k * a.Hs + slot) * 128; ld = a.ldq; r0 = 0;
            } else {
                dst = a.kc + ((int64_t)s * a.Hks + (slot - a.Hs)) * 128; ld = a.ldk; r0 = a.row0;
            }
#pragma unroll 4
            for (int it = 0; it < 16; ++it) {           // 4 rows of 16 lanes x 16 bytes per store
                const int r = w * 64 + it * 4 + (lane >> 4);
                const int c = (lane & 15) * 8;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg.lds + r * StagedRows16<BM>::PITCH + c0 + c);
                if (t0 + r < a.T) *reinterpret_cast<u32x4*>(dst + (r0 + t0 + r) * ld + c) = v;
            }
        } else {
            // V transposed: row (kv head, feature), sequence positions along
            // the row, each 32-position group stored as 4 chunks of 8 where
            // chunk j holds positions 4j..4j+3 and 16+4j..16+4j+3 (the order
            // the attention's P.V step consumes them); a lane gathers one
            // chunk of one feature
            const int64_t vrow0 = ((int64_t)s * a.Hks + (slot - a.Hs - a.Hks)) * 128;
#pragma unroll 2
            for (int it = 0; it < 16; ++it) {
                const int item = it * 256 + (int)threadIdx.x;
                const int c = item & 127, q = item >> 7;     // q = 4 * group + j
                const int r32 = (q >> 2) * 32, j = q & 3;
                if (t0 + r32 >= a.T) continue;          // T is a multiple of 32: a group is all in or all out
                uint16_t v[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = stg.lds[(r32 + 4 * j + e) * StagedRows16<BM>::PITCH + c0 + c];
                    v[4 + e] = stg.lds[(r32 + 16 + 4 * j + e) * StagedRows16<BM>::PITCH + c0 + c];
                }
                const u32x4 o = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                                 v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
                *reinterpret_cast<u32x4*>(a.vt + (vrow0 + c) * a.ldv + a.row0 + t0 + 8 * q) = o;
            }
        }
    }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_pack_qkv_bf16(const void* wq, const void* wk, const void* wv, void* dst, const int32_t* order,
                                int64_t rec_elems, int d, int H, int Hkv, int dh, int P, hipStream_t st) {
    const int Fq = H / P * dh, Fk = Hkv / P * dh;
    const int64_t chunks = (int64_t)(Fq + 2 * Fk) * d / 8;
    dim3 g((unsigned)std::min<int64_t>((chunks + 255) / 256, 4096), P);
    hipLaunchKernelGGL(pack_qkv_bf16, g, dim3(256), 0, st, (const uint16_t*)wq, (const uint16_t*)wk,
                       (const uint16_t*)wv, (uint16_t*)dst, order, rec_elems, d, H * dh, Hkv * dh, Fq, Fk, chunks);
    return hipGetLastError();
}

hipError_t launch_qkv(const ProjArgs& a, hipStream_t st) {
    const int fqkv = (a.Hs + 2 * a.Hks) * 128;
    if (fqkv % 256 || a.d % 64) return hipErrorInvalidValue;
    const int n_ft_shard = fqkv / 256, n_tt = (a.T + 255) / 256;
    const dim3 grid((unsigned)(a.P * n_ft_shard * n_tt));
    const bool buf = (int64_t)a.T * a.d * 2 < (int64_t(1) << 31) && (int64_t)a.d * 512 < (int64_t(1) << 31);
    if (buf) hipLaunchKernelGGL((qkv_w16<true>), grid, dim3(256), 0, st, a, n_ft_shard, n_tt);
    else hipLaunchKernelGGL((qkv_w16<false>), grid, dim3(256), 0, st, a, n_ft_shard, n_tt);
    return hipGetLastError();
}


}  // namespace tsp
