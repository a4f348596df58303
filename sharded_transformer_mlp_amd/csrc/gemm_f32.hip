// fp32 kernels of the sharded MLP: v_mfma_f32_16x16x4_f32 over LDS tiles, any
// shape (ragged edges are zero-filled in LDS and masked at the store).
//
// Used for fp32 storage (the parity-grade path). Same schedule as the bf16
// path: gate/up (or first-matrix) products per shard with the activation
// applied on the shard's own columns ("Tensor Parallelism: Splitting the
// Math", section "Why the column-then-row split": the nonlinearity is exact on
// a shard's own columns), then the down products accumulated over the shards
// in ring order into an fp32 Y ("Folding Tensor and Sequence Parallelism
// ...", Abstract: partial outputs accumulate locally).
// Per-shard fp32 record: [gate d x F][up d x F][down F x d], row-major
// (GeLU: [A d x F][B F x d]); records and the hidden columns of the
// workspace are stored in ring order, record k holding shard order[k].
//
// Both products put output features on the MFMA rows and tokens on its
// columns: a workgroup tile is 64 features x 64 tokens, four waves of 32 x 32
// (2 x 2 blocks of 16 x 16), 32 reduction indices per LDS stage. When the
// output has few tiles (the parity-sized shapes), the down product's
// reduction is split into up to 16 groups: group g takes the same sub-range
// of every ring step's hidden indices and writes an fp32 partial, and the
// partials are added in group order into Y (deterministic). For
// v_mfma_f32_16x16x4_f32 lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// and receives D[4 (l / 16) + r][l % 16], r = 0..3: four consecutive features
// of one token.
#include "common.h"
#include "launch.h"

namespace tsp {

constexpr int F32_MT = 64;   // features per workgroup tile
constexpr int F32_NT = 64;   // tokens per workgroup tile
constexpr int F32_KT = 32;   // reduction indices per stage

// Hidden indices per reduction group of a split down product: a multiple of
// the stage depth (the last group may be shorter).
__host__ __device__ inline int f32_split_chunk(int F, int split) {
    const int c = (F + split - 1) / split;
    return (c + F32_KT - 1) / F32_KT * F32_KT;
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Stage loads go through registers so that the next stage's global loads are
// in flight while the current stage's MFMAs run: fetch_* loads a thread's
// share (8 values), put_* writes it to LDS. Shares: element i = tid + 256 j.
constexpr int F32_PER = F32_KT * F32_MT / 256;          // values per thread per tile (8)
static_assert(F32_KT * F32_MT == F32_NT * F32_KT, "tile sizes");

// A k-major weight tile ws[k][feature] (k < F32_KT, feature < F32_MT) from a
// row-major matrix w (rows = reduction index, ld columns), zero outside
// [k_lim) x [f_lim).
__device__ __forceinline__ void fetch_w(float (&v)[F32_PER], const float* __restrict__ w, int64_t ld, int k0,
                                        int k_lim, int c0, int f_lim) {
#pragma unroll
    for (int j = 0; j < F32_PER; ++j) {
        const int i = threadIdx.x + 256 * j, r = i / F32_MT, c = i % F32_MT;
        const int k = k0 + r, fc = c0 + c;
        v[j] = (k < k_lim && fc < f_lim) ? w[(int64_t)k * ld + fc] : 0.f;
    }
}
__device__ __forceinline__ void put_w(float (*ws)[F32_MT + 4], const float (&v)[F32_PER]) {
#pragma unroll
    for (int j = 0; j < F32_PER; ++j) {
        const int i = threadIdx.x + 256 * j;
        ws[i / F32_MT][i % F32_MT] = v[j];
    }
}
// A token tile xs[token][k] from a row-major activation matrix (rows =
// tokens, ld columns, the stage's reduction indices at col0 + k0..).
__device__ __forceinline__ void fetch_x(float (&v)[F32_PER], const float* __restrict__ x, int64_t ld, int64_t col0,
                                        int t0, int T, int k0, int k_lim) {
#pragma unroll
    for (int j = 0; j < F32_PER; ++j) {
        const int i = threadIdx.x + 256 * j, r = i / F32_KT, c = i % F32_KT;
        const int tok = t0 + r, k = k0 + c;
        v[j] = (tok < T && k < k_lim) ? x[(int64_t)tok * ld + col0 + k] : 0.f;
    }
}
__device__ __forceinline__ void put_x(float (*xs)[F32_KT + 1], const float (&v)[F32_PER]) {
#pragma unroll
    for (int j = 0; j < F32_PER; ++j) {
        const int i = threadIdx.x + 256 * j;
        xs[i / F32_KT][i % F32_KT] = v[j];
    }
}

template <int ACT>
__global__ __launch_bounds__(256) void gateup_f32(F32Args a) {
    constexpr int NM = ACT == 1 ? 2 : 1;                 // weight matrices: gate and up, or A
    __shared__ float xs[F32_NT][F32_KT + 1];
    __shared__ float ws[NM][F32_KT][F32_MT + 4];
    poison_lds(xs, sizeof(xs));
    poison_lds(ws, sizeof(ws));
    const int s = blockIdx.z;                            // ring step = packed record
    const int c0 = blockIdx.x * F32_MT;                  // first local hidden column
    const int t0 = blockIdx.y * F32_NT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t dF = (int64_t)a.d * a.F;
    const float* rec = a.packed + (int64_t)s * a.shard_elems;
    f32x4 acc[NM][2][2];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float xv[F32_PER], wv[NM][F32_PER];
    fetch_x(xv, a.x, a.d, 0, t0, a.T, 0, a.d);
#pragma unroll
    for (int m = 0; m < NM; ++m) fetch_w(wv[m], rec + m * dF, a.F, 0, a.d, c0, a.F);
    for (int k0 = 0; k0 < a.d; k0 += F32_KT) {
        put_x(xs, xv);
#pragma unroll
        for (int m = 0; m < NM; ++m) put_w(ws[m], wv[m]);
        __syncthreads();
        if (k0 + F32_KT < a.d) {                         // the next stage's loads, in flight during the MFMAs
            fetch_x(xv, a.x, a.d, 0, t0, a.T, k0 + F32_KT, a.d);
#pragma unroll
            for (int m = 0; m < NM; ++m) fetch_w(wv[m], rec + m * dF, a.F, k0 + F32_KT, a.d, c0, a.F);
        }
#pragma unroll
        for (int ks = 0; ks < F32_KT / 4; ++ks) {
            const int kk = ks * 4 + (lane >> 4);
            float bx[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) bx[j] = xs[wn * 32 + j * 16 + (lane & 15)][kk];
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float aw = ws[m][kk][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[m][i][j] = mfma_f32(aw, bx[j], acc[m][i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tok = t0 + wn * 32 + j * 16 + (lane & 15);
            if (tok >= a.T) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hc = c0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
                if (hc < a.F) {
                    const float h = (ACT == 1) ? silu_f(acc[0][i][j][r]) * acc[NM - 1][i][j][r]
                                               : gelu_tanh_f(acc[0][i][j][r]);
                    a.h[(int64_t)tok * a.f + (int64_t)s * a.F + hc] = h;
                }
            }
        }
}

__global__ __launch_bounds__(256) void down_f32(F32Args a) {
    __shared__ float hs[F32_NT][F32_KT + 1];
    __shared__ float ds[F32_KT][F32_MT + 4];
    poison_lds(hs, sizeof(hs));
    poison_lds(ds, sizeof(ds));
    const int n0 = blockIdx.x * F32_MT;                  // first output feature
    const int t0 = blockIdx.y * F32_NT;
    const int g = blockIdx.z;                            // reduction group (split > 1)
    const int kchunk = f32_split_chunk(a.F, a.split);
    const int kg0 = g * kchunk, kg1 = min(a.F, kg0 + kchunk);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t down_off = (a.swiglu ? 2 : 1) * (int64_t)a.d * a.F;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stages: ring steps in order (records and H columns in ring order), each
    // the group's hidden sub-range in F32_KT slices; the next stage's loads
    // are in flight during the current stage's MFMAs
    const int per_step = (kg1 - kg0 + F32_KT - 1) / F32_KT;
    const int n_stages = a.P * per_step;
    float hv[F32_PER], dv[F32_PER];
    auto fetch = [&](int st) {
        const int step = st / per_step, k0 = kg0 + (st - step * per_step) * F32_KT;
        const float* wd = a.packed + (int64_t)step * a.shard_elems + down_off;   // F x d
        fetch_x(hv, a.h, a.f, (int64_t)step * a.F, t0, a.T, k0, kg1);
        fetch_w(dv, wd, a.d, k0, kg1, n0, a.d);
    };
    if (n_stages > 0) fetch(0);
    for (int st = 0; st < n_stages; ++st) {
        put_x(hs, hv);
        put_w(ds, dv);
        __syncthreads();
        if (st + 1 < n_stages) fetch(st + 1);
#pragma unroll
        for (int ks = 0; ks < F32_KT / 4; ++ks) {
            const int kk = ks * 4 + (lane >> 4);
            float bh[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) bh[j] = hs[wn * 32 + j * 16 + (lane & 15)][kk];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float aw = ds[kk][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f32(aw, bh[j], acc[i][j]);
            }
        }
        __syncthreads();
    }
    float* out = a.split > 1 ? a.part + (int64_t)g * a.T * a.d : a.y;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tok = t0 + wn * 32 + j * 16 + (lane & 15);
            if (tok >= a.T) continue;
            const int n = n0 + wm * 32 + i * 16 + 4 * (lane >> 4);
            float* yrow = out + (int64_t)tok * a.d;
            if (n + 3 < a.d && (a.d & 3) == 0) {
                *reinterpret_cast<f32x4*>(yrow + n) = acc[i][j];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < a.d) yrow[n + r] = acc[i][j][r];
            }
        }
}

// y[i] = sum over groups g = 0.. of part[g][i], in group order.
__global__ __launch_bounds__(256) void reduce_f32(const float* __restrict__ part, int split, int64_t n,
                                                  float* __restrict__ y) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float s = part[i];
        for (int g = 1; g < split; ++g) s += part[(int64_t)g * n + i];
        y[i] = s;
    }
}

int choose_f32_split(int T, int d, int F) {
    const int64_t tiles = (int64_t)((d + F32_MT - 1) / F32_MT) * ((T + F32_NT - 1) / F32_NT);
    int s = 1;
    while (s < 16 && tiles * s * 2 <= 256 && f32_split_chunk(F, s * 2) * (s * 2 - 1) < F) s *= 2;
    return s;
}

int64_t f32_split_bytes(int64_t T_max, int d, int F) {
    int64_t most = 0;
    for (int64_t t = F32_NT; t < T_max + F32_NT; t += F32_NT) {
        const int64_t T = t < T_max ? t : T_max;
        const int s = choose_f32_split((int)T, d, F);
        if (s > 1 && s * T * d * 4 > most) most = s * T * d * 4;
    }
    return most;
}

hipError_t launch_gateup_f32(const F32Args& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.F + F32_MT - 1) / F32_MT), (unsigned)((a.T + F32_NT - 1) / F32_NT), (unsigned)a.P);
    if (a.swiglu)
        hipLaunchKernelGGL(gateup_f32<1>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(gateup_f32<2>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_down_f32(const F32Args& a, hipStream_t st) {
    if (a.split < 1 || a.split > 16 || (a.split > 1 && !a.part)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.d + F32_MT - 1) / F32_MT), (unsigned)((a.T + F32_NT - 1) / F32_NT),
                    (unsigned)a.split);
    hipLaunchKernelGGL(down_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_reduce_f32(const float* part, int split, int64_t n, float* y, hipStream_t st) {
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 2048);
    hipLaunchKernelGGL(reduce_f32, dim3((unsigned)blocks), dim3(256), 0, st, part, split, n, y);
    return hipGetLastError();
}

}  // namespace tsp
