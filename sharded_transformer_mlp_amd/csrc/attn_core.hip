// Causal (or full) softmax attention of one TSP rank's queries over the
// sequence-wide key/value context, all head groups in one launch (gfx950).
// Built on its own with MFMA results in vector registers
// (-mllvm -amdgpu-mfma-vgpr-form): the softmax reads every score, and with
// accumulation-register results each score was first copied out.
//
// "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
// Training & Inference", Abstract: the ranks rebuild the full context through
// a sequence-wise key/value exchange; "Tensor Parallelism: Splitting the Math",
// section "Why the column-then-row split - and what happens in attention":
// a head's attention runs locally on the device that owns the head.
#include "attn.h"
#include "common.h"
#include "w16.h"

namespace tsp {

// ------------------------------------------------------------------ attention
//
// Workgroup: 16 / QT waves, each 16 QT queries of one head against 64-key
// blocks of the context; the waves share the key/value head (hw heads x qs
// 64-query sub-tiles, hw * qs = 4), so one K tile and one V tile in LDS serve
// them all.
// With v_mfma_f32_16x16x32_f16 a wave computes S^T = K Q^T (keys as rows:
// lane l holds 4 consecutive keys of query l % 16), so a query's softmax
// statistics sit in one lane column and reduce with two cross-lane steps; the
// probabilities then feed O^T = V^T P^T as the B operand straight from the
// registers: within a 32-key step, lane group g = l / 16 takes keys 4g..4g+3
// and 16+4g..16+4g+3 (its own S^T values), and the value context stores each
// 32-position group in that order (16-byte chunk g = those 8 positions), so
// the V^T fragment is one 16-byte read. Scores are kept in log2 units (scale log2(e)/sqrt(dh))
// and exponentiated with v_exp_f32.
//
// Context tiles reach LDS by DMA (buffer loads into LDS, 16 bytes per lane;
// K in three buffers, V^T in two): K as 64 rows of 256 bytes with the 16-byte
// chunk c of row r at c ^ (r & 15), V^T as 128 rows of 128 bytes with chunk c
// at c ^ ((r >> 1) & 7); both make the fragment reads of 16 rows hit distinct
// banks. All buffers (and the restart flag) live in one LDS array: with one
// array per operand the compiler tells the arrays apart and, before every
// fragment read, waits for the newest DMA into that array, i.e. for the next
// tile's prefetch, in the middle of the current tile (13 % of the kernel's
// time). The loop orders its reads itself: every tile ends with vmcnt(0) and
// a barrier, and a buffer is reloaded only after the barrier that follows its
// last read.
//
// Softmax with a fixed exponent reference per query instead of a running
// maximum: the first block's maximum. O / l does not depend on the reference,
// so the accumulators are never rescaled (rescaling them, 128 accumulation
// registers, cost more than the exponentials). The probabilities enter the
// P.V product as fp16, whose range bounds them: a block whose scores exceed
// the reference by more than ~16 log2 units (a probability above 65504) sets a
// workgroup flag; the workgroup then finds every query's true maximum in a
// pass over the keys and starts again with it (rare: logits 11 nats above the
// first block's largest).
//
// Precision: queries, keys and values arrive as fp16 from the projection and
// the probabilities are rounded to fp16 (11 significant bits: each rounding
// a relative 2^-11 at most, 8x finer than bf16); the fp32 output is rounded
// once, to bf16, for the output projection.

constexpr int ATT_KROW = 128;   // K tile row (elements)
constexpr int ATT_VROW = 64;    // V^T tile row (elements)
constexpr int ATT_K_ELEMS = 3 * 64 * ATT_KROW;   // three K tiles
constexpr int ATT_V_ELEMS = 2 * 128 * ATT_VROW;  // two V^T tiles

__device__ __forceinline__ void att_vm_zero() {
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
}

__device__ inline f16x8 att_pack8(f32x4 lo, f32x4 hi) {
    f16x8 r;
    r[0] = static_cast<_Float16>(lo[0]); r[1] = static_cast<_Float16>(lo[1]);
    r[2] = static_cast<_Float16>(lo[2]); r[3] = static_cast<_Float16>(lo[3]);
    r[4] = static_cast<_Float16>(hi[0]); r[5] = static_cast<_Float16>(hi[1]);
    r[6] = static_cast<_Float16>(hi[2]); r[7] = static_cast<_Float16>(hi[3]);
    return r;
}

// QT query tiles of 16 per wave, 16 / QT waves per workgroup: 64 query rows
// per four waves either way. QT = 2 is kept: two waves per SIMD (230 vector
// registers each), one wave's softmax and fragment reads beside the other's
// MFMAs, measured 4 % faster than QT = 4 (one wave per SIMD, 128 query rows
// per SIMD in flight); each K or V^T fragment read then feeds two MFMAs
// instead of four.
constexpr int QT = 2;

__global__ __launch_bounds__(64 * (16 / QT)) void attn_fwd(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint16_t lds[ATT_K_ELEMS + ATT_V_ELEMS + 128];
    uint16_t* const k_lds = lds;
    uint16_t* const v_lds = lds + ATT_K_ELEMS;
    int* const restart_flag = reinterpret_cast<int*>(lds + ATT_K_ELEMS + ATT_V_ELEMS);
    poison_lds(lds, (ATT_K_ELEMS + ATT_V_ELEMS) * 2);

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
    const int q0 = q_wg + (w / a.hw) * (16 * QT);        // first query of the wave
    const int64_t qo_col = ((int64_t)k * a.Hs + hl) * 128;

    // Q^T fragments (B operand): query t*16 + n16, head dims ks*32 + 8g .. + 7
    f16x8 qf[QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int row = min(q0 + t * 16 + n16, a.T - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qf[t][ks] = *reinterpret_cast<const f16x8*>(a.q + (int64_t)row * a.ldq + qo_col + ks * 32 + 8 * g);
    }
    // (the projection stored the queries scaled by log2(e)/sqrt(dh): the
    // scores come out in log2 units)

    const int q_hi = min(a.T, q_wg + 64 * a.qs);         // queries of the workgroup end here
    const int kend = a.causal ? min(a.S, a.row0 + q_hi) : a.S;
    const int nkb = (kend + 63) / 64;
    const int qpos0 = a.row0 + q0;                       // the wave's first query position

    // DMA of one context block into buffer `buf`: 4 K and 4 V^T instructions
    // per wave, each 1 KiB of LDS (4 K rows or 8 V^T rows). Buffer loads: the
    // block's base is scalar, a lane's offset (fixed for the whole loop) 32-bit.
    int k_off[QT], v_off[QT];
#pragma unroll
    for (int i = 0; i < QT; ++i) {
        const int j = w * QT + i;
        const int kr = j * 4 + (lane >> 4), kc = (lane & 15) ^ (kr & 15);
        k_off[i] = (int)((kr * a.ldk + kc * 8) * 2);
        const int vr = j * 8 + (lane >> 3), vc = (lane & 7) ^ ((vr >> 1) & 7);
        v_off[i] = (int)((vr * a.ldv + vc * 8) * 2);
    }
    auto load_k = [&](int kb, int buf) {
        const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.kc + (int64_t)kb * 64 * a.ldk + kv_col), (short)0, 0x7fffffff, kRawBufferWord3);
#pragma unroll
        for (int i = 0; i < QT; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (TSP_LDS void*)(k_lds + buf * 64 * ATT_KROW + (w * QT + i) * 512), 16, k_off[i],
                                                     0, 0, 0);
    };
    auto load_v = [&](int kb, int buf) {
        const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.vt + kv_col * a.ldv + kb * 64), (short)0, 0x7fffffff, kRawBufferWord3);
#pragma unroll
        for (int i = 0; i < QT; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (TSP_LDS void*)(v_lds + buf * 128 * ATT_VROW + (w * QT + i) * 512), 16, v_off[i],
                                                     0, 0, 0);
    };

    f32x4 o[8][QT];
    float m[QT], l[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) m[t] = -INFINITY;

    // The key stream runs in 32-key halves of the 64-key tiles: half h of a
    // tile is its key tiles 2h, 2h+1 (16 keys each) and the P.V step ks2 = h.
    // K fragments of one 32-dim step of that half (from buffer `buf`), and
    // the step's 8 MFMAs of S^T = K Q^T (2 key tiles x 4 query tiles); ks == 0
    // starts the accumulators.
    auto read_k = [&](int ks, int buf, int h, f16x8 (&kf)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
            kf[u] = *reinterpret_cast<const f16x8*>(
                k_lds + buf * 64 * ATT_KROW + ((2 * h + u) * 16 + n16) * ATT_KROW + ((4 * ks + g) ^ n16) * 8);
    };
    // init[t]: the accumulators' start for ks == 0 (zero, or minus the
    // query's reference so that the scores come out already shifted)
    auto s_mfma = [&](int ks, const f16x8 (&kf)[2], f32x4 (&sc)[2][QT], const float (&init)[QT]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < QT; ++t)
                sc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    kf[u], qf[t][ks], ks == 0 ? f32x4{init[t], init[t], init[t], init[t]} : sc[u][t], 0, 0, 0);
    };
    const float zero_init[QT] = {};
    // all four steps, each step's K fragments read one step ahead
    auto s_half = [&](int buf, int h, f32x4 (&sc)[2][QT]) {
        f16x8 kf[2][2];
        read_k(0, buf, h, kf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) read_k(ks + 1, buf, h, kf[(ks + 1) & 1]);
            s_mfma(ks, kf[ks & 1], sc, zero_init);
        }
    };
    // keys past the query (causal) or past the context end get -inf
    auto apply_mask = [&](int kb, int h, f32x4 (&sc)[2][QT]) {
        const int kbase = kb * 64 + 32 * h;
        const int lim_s = a.S - kbase - 4 * g;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const int lim_q = a.causal ? qpos0 + t * 16 + n16 - kbase - 4 * g + 1 : 1 << 30;
            const int lim = min(lim_q, lim_s);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[u][t][i] = u * 16 + i < lim ? sc[u][t][i] : -INFINITY;
        }
    };
    // a query's maximum over the half in log2 units: the lane's 8 keys, then
    // the 4 lane groups (the scale is positive, so it commutes with the maximum)
    auto half_max = [&](const f32x4 (&sc)[2][QT], int t) {
        float mx = sc[0][t][0];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[u][t][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        return fmaxf(mx, __shfl_xor(mx, 32));
    };
    // probabilities of query tile t against the fixed reference, added into
    // the lane's partial sum and packed as the B operand of the P.V step
    auto softmax_t = [&](f32x4 (&sc)[2][QT], int t, f16x8 (&pb)[QT], bool shifted) {
        const float ref = m[t] == -INFINITY ? 0.f : m[t];
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pr = __builtin_amdgcn_exp2f(shifted ? sc[u][t][i] : sc[u][t][i] - ref);
                sc[u][t][i] = pr;
                ls += pr;
            }
        l[t] += ls;
        pb[t] = att_pack8(sc[0][t], sc[1][t]);
    };
    // V^T fragment dt of half h (the 8 keys lane group g multiplies)
    auto read_v = [&](int buf, int h, int dt) {
        const int r = dt * 16 + n16;
        return *reinterpret_cast<const f16x8*>(v_lds + buf * 128 * ATT_VROW + r * ATT_VROW + ((4 * h + g) ^ ((r >> 1) & 7)) * 8);
    };
    // O^T += V^T P^T over half h of the V^T tile in buffer `buf`, fragments
    // read two ahead; vf holds the first two (read early by the caller)
    auto pv = [&](int buf, int h, const f16x8 (&pb)[QT], f16x8 (&vf)[3]) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            if (dt + 2 < 8) vf[(dt + 2) % 3] = read_v(buf, h, dt + 2);
#pragma unroll
            for (int t = 0; t < QT; ++t)
                o[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt % 3], pb[t], o[dt][t], 0, 0, 0);
        }
    };
    // half n+1's scores on the matrix cores while the VALU turns half n's
    // into probabilities, then half n's P.V. That first part runs at raised
    // wave priority and the P.V MFMAs at the normal one: when the SIMD's other
    // wave is in its P.V burst, this wave's score MFMAs, fragment reads and
    // softmax (the chain the next P.V waits on) issue first (measured 1 %
    // faster, same results; the reverse, raised priority over the P.V burst,
    // 1 % slower). Each query tile's softmax follows the second of its two
    // score steps and the first V^T fragments are read two steps before the
    // P.V (measured 0.6-0.8 % faster than after the first step and one step
    // before)
    // cur_shifted: cur's scores already have the reference subtracted; the
    // next half's always do (init = minus the reference)
    auto step = [&](int kbuf_next, int h_next, f32x4 (&cur)[2][QT], f32x4 (&nxt)[2][QT], int vbuf, int h,
                    bool cur_shifted, const float (&negref)[QT]) {
        f16x8 pb[QT], kf[2][2], vf[3];
        __builtin_amdgcn_s_setprio(1);
        read_k(0, kbuf_next, h_next, kf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) read_k(ks + 1, kbuf_next, h_next, kf[(ks + 1) & 1]);
            if (ks == 2) {
                vf[0] = read_v(vbuf, h, 0);
                vf[1] = read_v(vbuf, h, 1);
            }
            s_mfma(ks, kf[ks & 1], nxt, negref);
            if (ks % (4 / QT) == (4 / QT) - 1) softmax_t(cur, ks / (4 / QT), pb, cur_shifted);
        }
        __builtin_amdgcn_s_setprio(0);
        pv(vbuf, h, pb, vf);
    };
    auto last_step = [&](f32x4 (&cur)[2][QT], int vbuf, int h, bool shifted) {
        f16x8 pb[QT], vf[3];
        vf[0] = read_v(vbuf, h, 0);
        vf[1] = read_v(vbuf, h, 1);
#pragma unroll
        for (int t = 0; t < QT; ++t) softmax_t(cur, t, pb, shifted);
        pv(vbuf, h, pb, vf);
    };

    // Tiles every query of the workgroup sees in full (no mask) come first and
    // run software-pipelined (K tiles in 3 buffers, V^T tiles in 2: tile kb's
    // K is read in its first half and by the previous tile's second half). The
    // masked tiles (the diagonal, the context end) run one at a time after.
    const int first_q = a.row0 + q_wg;                   // the workgroup's first query position
    int n_full = a.causal ? (first_q + 1) / 64 : a.S / 64;
    n_full = min(n_full, min(nkb, a.S / 64));

    for (int attempt = 0; attempt < 2; ++attempt) {
        if (tid == 0) *restart_flag = 0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int t = 0; t < QT; ++t) o[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < QT; ++t) l[t] = 0.f;

        if (n_full > 0) {
            f32x4 sa[2][QT], sb[2][QT];
            load_k(0, 0);
            load_v(0, 0);
            load_k(min(1, nkb - 1), 1);
            att_vm_zero();
            __syncthreads();
            s_half(0, 0, sa);
            if (attempt == 0) {
#pragma unroll
                for (int t = 0; t < QT; ++t) m[t] = half_max(sa, t);   // the reference
            }
            // every later half's scores start from minus the reference
            float negref[QT];
#pragma unroll
            for (int t = 0; t < QT; ++t) negref[t] = -m[t];
            int kb = 0;
            if (n_full > 1) {                            // tile 0: its first half's scores are not shifted
                load_k(min(2, nkb - 1), 2);
                load_v(1, 1);
                step(0, 1, sa, sb, 0, 0, false, negref);
                step(1, 0, sb, sa, 0, 1, true, negref);
                att_vm_zero();
                __syncthreads();
                kb = 1;
            }
            for (; kb + 1 < n_full; ++kb) {
                // buffer (kb+2)%3 held tile kb-1's K, (kb+1)&1 tile kb-1's V^T:
                // both last read before the previous barrier
                load_k(min(kb + 2, nkb - 1), (kb + 2) % 3);
                load_v(kb + 1, (kb + 1) & 1);
                step(kb % 3, 1, sa, sb, kb & 1, 0, true, negref);        // scores of this tile's second half
                step((kb + 1) % 3, 0, sb, sa, kb & 1, 1, true, negref);  // scores of the next tile's first half
                att_vm_zero();
                __syncthreads();
            }
            step(kb % 3, 1, sa, sb, kb & 1, 0, kb > 0, negref);
            last_step(sb, kb & 1, 1, true);
            __syncthreads();                             // every read of the buffers is done
        }
        // masked tiles, one at a time
        for (int kb = n_full; kb < nkb; ++kb) {
            load_k(kb, 0);
            load_v(kb, 0);
            att_vm_zero();
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 sc[2][QT];
                s_half(0, h, sc);
                apply_mask(kb, h, sc);
#pragma unroll
                for (int t = 0; t < QT; ++t)
                    if (m[t] == -INFINITY) m[t] = half_max(sc, t);   // the first keys set the reference
                last_step(sc, 0, h, false);
            }
            __syncthreads();
        }
        // a probability beyond fp16's range (above 65504: a score more than
        // ~16 log2 units above the reference) shows in the lane's partial sum,
        // which bounds every probability it adds up; an unneeded restart on
        // many large ones only costs time
        bool over = false;
#pragma unroll
        for (int t = 0; t < QT; ++t) over |= !(l[t] <= 65000.0f);
        if (__any(over)) *restart_flag = 1;
        __syncthreads();
        if (!*restart_flag) break;                        // same value in every wave
        // rare: take every query's true maximum over all keys, start again
        for (int kb = 0; kb < nkb; ++kb) {
            load_k(kb, 0);
            att_vm_zero();
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 sc[2][QT];
                s_half(0, h, sc);
                apply_mask(kb, h, sc);
#pragma unroll
                for (int t = 0; t < QT; ++t) m[t] = fmaxf(m[t], half_max(sc, t));
            }
            __syncthreads();                             // reads done before the next tile's DMA
        }
    }

    // normalise and store: lane holds O[query t*16 + n16][dims dt*16 + 4g .. + 3]
#pragma unroll
    for (int t = 0; t < QT; ++t) {
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

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
    const int64_t wgs = (int64_t)a.n_qt * a.P * a.Hks * a.n_hq;
    if (wgs < 1 || wgs > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_fwd, dim3((unsigned)wgs), dim3(64 * (16 / QT)), 0, st, a);
    return hipGetLastError();
}

}  // namespace tsp
