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
//   qkv_w16        the projection: the MLP's shape-6 pipeline (w16.h) over
//                  the records with a plain epilogue that sends each 128-column
//                  head to its place: Q to the rank's query buffer, K rows to
//                  the key context, V transposed to the value context.
//   attn_fwd       flash-style attention, one workgroup per (64 .. 256
//                  queries, up to 4 heads of one key/value head); the output
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
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE];
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
    // 128-feature half, one head, to its destination
    StagedRows16<BM> stg{lds};
    stage_barrier();
    const int fsub = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const f32x4 u = acc[i][j];
            stg.put4((wn * TN + j) * 16 + (lane & 15), (wm * TM + i) * 16 + fsub, pack4_bf16(u[0], u[1], u[2], u[3]));
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
            // the row; a lane gathers 8 consecutive tokens of one feature
            const int64_t vrow0 = ((int64_t)s * a.Hks + (slot - a.Hs - a.Hks)) * 128;
#pragma unroll 2
            for (int it = 0; it < 16; ++it) {
                const int item = it * 256 + (int)threadIdx.x;
                const int c = item & 127, r8 = (item >> 7) * 8;
                if (t0 + r8 >= a.T) continue;           // T is a multiple of 8: a chunk is all in or all out
                uint16_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = stg.lds[(r8 + e) * StagedRows16<BM>::PITCH + c0 + c];
                const u32x4 o = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                                 v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
                *reinterpret_cast<u32x4*>(a.vt + (vrow0 + c) * a.ldv + a.row0 + t0 + r8) = o;
            }
        }
    }
}

// ------------------------------------------------------------------ attention
//
// Workgroup: 4 waves, each 64 queries of one head against 64-key blocks of
// the context; the 4 waves share the key/value head (hw heads x qs query
// sub-tiles, hw * qs = 4), so one K tile and one V tile in LDS serve them all.
// With v_mfma_f32_16x16x32_bf16 a wave computes S^T = K Q^T (keys as rows:
// lane l holds 4 consecutive keys of query l % 16), so a query's softmax
// statistics sit in one lane column and reduce with two cross-lane steps; the
// probabilities then feed O^T = V^T P^T as the B operand straight from the
// registers: within a 32-key step, lane group g = l / 16 takes keys 4g..4g+3
// and 16+4g..16+4g+3 (its own S^T values), and the V^T fragment is read with
// the same key order. Scores are kept in log2 units (scale log2(e)/sqrt(dh))
// and exponentiated with v_exp_f32.
//
// Context tiles reach LDS by DMA (global_load_lds, 16 bytes per lane, two
// buffers): K as 64 rows of 256 bytes with the 16-byte chunk c of row r at
// c ^ (r & 15), V^T as 128 rows of 128 bytes with chunk c at c ^ ((r >> 1) & 7);
// both make the fragment reads of 16 rows hit distinct banks.
//
// Softmax with a fixed exponent reference per query instead of a running
// maximum: the first block's maximum. O / l does not depend on the reference,
// and probabilities up to 2^64 (a later block's scores up to 64 above it, in
// log2 units) are exact enough in fp32 and bf16, so the accumulators are never
// rescaled (rescaling them, 128 accumulation registers, cost more than the
// exponentials). A block that exceeds the reference by more than that sets a
// workgroup flag; the workgroup then finds every query's true maximum in a
// pass over the keys and starts again with it (rare: logits 44 nats apart).

constexpr int ATT_KROW = 128;   // K tile row (elements)
constexpr int ATT_VROW = 64;    // V^T tile row (elements)
constexpr float ATT_HEADROOM = 64.0f;

__device__ __forceinline__ void att_vm_zero() {
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
}

__device__ inline bf16x8 att_pack8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
    r[0] = static_cast<__bf16>(lo[0]); r[1] = static_cast<__bf16>(lo[1]);
    r[2] = static_cast<__bf16>(lo[2]); r[3] = static_cast<__bf16>(lo[3]);
    r[4] = static_cast<__bf16>(hi[0]); r[5] = static_cast<__bf16>(hi[1]);
    r[6] = static_cast<__bf16>(hi[2]); r[7] = static_cast<__bf16>(hi[3]);
    return r;
}

__global__ __launch_bounds__(256) void attn_fwd(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][64 * ATT_KROW];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][128 * ATT_VROW];
    poison_lds(k_lds, sizeof(k_lds));
    poison_lds(v_lds, sizeof(v_lds));

    // heaviest query tiles first; consecutive workgroups (different XCDs)
    // take different key/value heads, so each XCD's L2 streams few contexts
    const int per_qt = a.P * a.Hks * a.n_hq;
    const int lin = blockIdx.x;
    const int qt = a.n_qt - 1 - lin / per_qt;
    int rem = lin - (lin / per_qt) * per_qt;
    const int hq = rem % a.n_hq;
    rem /= a.n_hq;
    const int jl = rem % a.Hks;
    const int k = rem / a.Hks;
    const int s = a.order[k];
    const int64_t kv_col = ((int64_t)s * a.Hks + jl) * 128;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.Hs / a.Hks;
    const int hl = jl * G + hq * a.hw + (w % a.hw);
    const int q_wg = qt * 64 * a.qs;                     // first query of the workgroup
    const int q0 = q_wg + (w / a.hw) * 64;               // first query of the wave
    const int64_t qo_col = ((int64_t)k * a.Hs + hl) * 128;

    // Q^T fragments (B operand): query t*16 + n16, head dims ks*32 + 8g .. + 7
    bf16x8 qf[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int row = min(q0 + t * 16 + n16, a.T - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qf[t][ks] = *reinterpret_cast<const bf16x8*>(a.q + (int64_t)row * a.ldq + qo_col + ks * 32 + 8 * g);
    }

    const int q_hi = min(a.T, q_wg + 64 * a.qs);         // queries of the workgroup end here
    const int kend = a.causal ? min(a.S, a.row0 + q_hi) : a.S;
    const int nkb = (kend + 63) / 64;
    const int qpos0 = a.row0 + q0;                       // the wave's first query position

    // DMA of one context block into buffer `buf`: 4 K and 4 V^T instructions
    // per wave, each 1 KiB of LDS (4 K rows or 8 V^T rows). Buffer loads: the
    // block's base is scalar, a lane's offset (fixed for the whole loop) 32-bit.
    int k_off[4], v_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = w * 4 + i;
        const int kr = j * 4 + (lane >> 4), kc = (lane & 15) ^ (kr & 15);
        k_off[i] = (int)((kr * a.ldk + kc * 8) * 2);
        const int vr = j * 8 + (lane >> 3), vc = (lane & 7) ^ ((vr >> 1) & 7);
        v_off[i] = (int)((vr * a.ldv + vc * 8) * 2);
    }
    auto load_kv = [&](int kb, int buf) {
        const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.kc + (int64_t)kb * 64 * a.ldk + kv_col), (short)0, 0x7fffffff, kRawBufferWord3);
        const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.vt + kv_col * a.ldv + kb * 64), (short)0, 0x7fffffff, kRawBufferWord3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = w * 4 + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (TSP_LDS void*)&k_lds[buf][j * 512], 16, k_off[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (TSP_LDS void*)&v_lds[buf][j * 512], 16, v_off[i], 0, 0, 0);
        }
    };

    __shared__ int restart_flag;
    f32x4 o[8][4];
    float m[4], l[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = -INFINITY;

    // S^T = K Q^T of the block in buffer `buf` for 4 key tiles x 4 query tiles,
    // masked (keys past the query when causal, past the context end; the
    // scale to log2 units is applied with the exponent); the K fragments of one 32-dim step are read while the
    // previous step's MFMAs run, the fences keeping the compiler from hoisting
    // all 16 reads (registers the loop cannot afford)
    auto scores = [&](int kb, int buf, f32x4 (&sc)[4][4]) {
        bf16x8 kf[2][4];
        auto read_k = [&](int ks, bf16x8 (&dst)[4]) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                dst[kt] = *reinterpret_cast<const bf16x8*>(
                    &k_lds[buf][(kt * 16 + n16) * ATT_KROW + ((4 * ks + g) ^ n16) * 8]);
        };
        read_k(0, kf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) read_k(ks + 1, kf[(ks + 1) & 1]);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    sc[kt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        kf[ks & 1][kt], qf[t][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[kt][t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int kbase = kb * 64;
        const bool masked = (a.causal && kbase + 63 > qpos0) || kbase + 64 > a.S;
        if (masked) {                                    // one branch per block, selects inside
            const int lim_s = a.S - kbase - 4 * g;       // key index within the lane's run must stay below
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // keys kbase + kt*16 + 4g + i visible to query qpos0 + t*16 + n16
                const int lim_q = a.causal ? qpos0 + t * 16 + n16 - kbase - 4 * g + 1 : 1 << 30;
                const int lim = min(lim_q, lim_s);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc[kt][t][i] = kt * 16 + i < lim ? sc[kt][t][i] : -INFINITY;
            }
        }
    };
    // a query's block maximum in log2 units: the lane's 16 keys, then the 4
    // lane groups (the scale is positive, so it commutes with the maximum)
    auto block_max = [&](const f32x4 (&sc)[4][4], int t) {
        float mx = sc[0][t][0];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kt][t][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        return fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    };

    for (int attempt = 0; attempt < 2; ++attempt) {
        if (tid == 0) restart_flag = 0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int t = 0; t < 4; ++t) o[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) l[t] = 0.f;
        load_kv(0, 0);
        att_vm_zero();
        __syncthreads();
        bool restart = false;
        for (int kb = 0; kb < nkb; ++kb) {
            const int cur = kb & 1;
            // the other buffer's last readers passed the previous barrier
            if (kb + 1 < nkb) load_kv(kb + 1, cur ^ 1);
            f32x4 sc[4][4];
            scores(kb, cur, sc);
            bool over = false;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float mx = block_max(sc, t);
                if (m[t] == -INFINITY) m[t] = mx;        // the first block sets the reference
                over |= mx > m[t] + ATT_HEADROOM;
                const float ref = m[t] == -INFINITY ? 0.f : m[t];
                float ls = 0.f;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][t][i], a.scale_log2, -ref));
                        sc[kt][t][i] = p;
                        ls += p;
                    }
                l[t] += ls;
            }
            if (__any(over)) restart_flag = 1;           // read by every wave after the barrier below

            // O^T += V^T P^T over two 32-key steps
            bf16x8 pb[2][4];
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
                for (int t = 0; t < 4; ++t) pb[ks2][t] = att_pack8(sc[2 * ks2][t], sc[2 * ks2 + 1][t]);
            __builtin_amdgcn_sched_barrier(0);
            auto read_v = [&](int ks2, int dt) {
                const int r = dt * 16 + n16, sw = (r >> 1) & 7, c = 4 * ks2 + (g >> 1);
                const uint16_t* vrow = &v_lds[cur][r * ATT_VROW + (g & 1) * 4];
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow + ((c ^ sw) * 8));
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (((c + 2) ^ sw) * 8));
                const u32x4 vv = {lo.x, lo.y, hi.x, hi.y};
                return __builtin_bit_cast(bf16x8, vv);
            };
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
                for (int dt = 0; dt < 8; dt += 2) {
                    const bf16x8 v0 = read_v(ks2, dt), v1 = read_v(ks2, dt + 1);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        o[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pb[ks2][t], o[dt][t], 0, 0, 0);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        o[dt + 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pb[ks2][t], o[dt + 1][t], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            att_vm_zero();                               // this wave's DMA of the next block landed
            __syncthreads();                             // everyone's landed, this block's reads are done
            if (restart_flag) { restart = true; break; } // same value in every wave
        }
        if (!restart) break;
        // rare: some query's scores rose more than the headroom above its
        // reference; take every query's true maximum over all blocks and
        // start again (a violation cannot recur with the true maximum)
        att_vm_zero();
        __syncthreads();
        for (int kb = 0; kb < nkb; ++kb) {
            load_kv(kb, 0);
            att_vm_zero();
            __syncthreads();
            f32x4 sc[4][4];
            scores(kb, 0, sc);
#pragma unroll
            for (int t = 0; t < 4; ++t) m[t] = fmaxf(m[t], block_max(sc, t));
            __syncthreads();                             // reads done before the next block's DMA
        }
    }

    // normalise and store: lane holds O[query t*16 + n16][dims dt*16 + 4g .. + 3]
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float lt = l[t];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const float inv = 1.0f / lt;
        const int row = q0 + t * 16 + n16;
        if (row < a.T) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f32x4 v = o[dt][t] * inv;
                *reinterpret_cast<uint2*>(a.o + (int64_t)row * a.ldq + qo_col + dt * 16 + 4 * g) =
                    pack4_bf16(v[0], v[1], v[2], v[3]);
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

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    const int64_t wgs = (int64_t)a.n_qt * a.P * a.Hks * a.n_hq;
    if (wgs < 1 || wgs > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_fwd, dim3((unsigned)wgs), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace tsp
