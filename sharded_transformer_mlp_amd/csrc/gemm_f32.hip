// fp32 kernels of the sharded MLP: LDS-tiled FMA, any shape.
//
// Used for fp32 storage (the parity-grade path). Same schedule as the bf16
// path: gate/up (or first-matrix) products per shard with the activation
// applied on the shard's own columns, then the down products accumulated
// over the shards in ring order into an fp32 Y.
// Per-shard fp32 record: [gate d x F][up d x F][down F x d], row-major
// (GeLU: [A d x F][B F x d]); records and the hidden columns of the
// workspace are stored in ring order, record k holding shard order[k].
#include "common.h"
#include "launch.h"

namespace tsp {

constexpr int FT = 32;   // tile edge (tokens, features, reduction)

template <int ACT>
__global__ __launch_bounds__(256) void gateup_f32(F32Args a) {
    __shared__ float xs[FT][FT + 1];
    __shared__ float gs[FT][FT + 1];
    __shared__ float us[FT][FT + 1];
    poison_lds(xs, sizeof(xs));
    poison_lds(gs, sizeof(gs));
    poison_lds(us, sizeof(us));
    const int s = blockIdx.z;                            // ring step = packed record
    const int c0 = blockIdx.x * FT;                      // local hidden column
    const int t0 = blockIdx.y * FT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t dF = (int64_t)a.d * a.F;
    const float* rec = a.packed + (int64_t)s * a.shard_elems;
    const float* wg = rec;                               // gate (SwiGLU only)
    const float* wu = (ACT == 1) ? rec + dF : rec;       // up, or A
    float g[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, u[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    for (int k0 = 0; k0 < a.d; k0 += FT) {
        for (int i = threadIdx.x; i < FT * FT; i += 256) {
            const int r = i / FT, c = i % FT;
            const int tok = t0 + r, k = k0 + c;
            xs[r][c] = (tok < a.T && k < a.d) ? a.x[(int64_t)tok * a.d + k] : 0.f;
            const int kr = k0 + r, hc = c0 + c;
            const bool ok = kr < a.d && hc < a.F;
            us[r][c] = ok ? wu[(int64_t)kr * a.F + hc] : 0.f;
            if (ACT == 1) gs[r][c] = ok ? wg[(int64_t)kr * a.F + hc] : 0.f;
        }
        __syncthreads();
        for (int k = 0; k < FT; ++k) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float xv = xs[ty * 2 + i][k];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    u[i][j] = fmaf(xv, us[k][tx * 2 + j], u[i][j]);
                    if (ACT == 1) g[i][j] = fmaf(xv, gs[k][tx * 2 + j], g[i][j]);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tok = t0 + ty * 2 + i;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int hc = c0 + tx * 2 + j;
            if (tok < a.T && hc < a.F) {
                const float h = (ACT == 1) ? silu_f(g[i][j]) * u[i][j] : gelu_tanh_f(u[i][j]);
                a.h[(int64_t)tok * a.f + (int64_t)s * a.F + hc] = h;
            }
        }
    }
}

__global__ __launch_bounds__(256) void down_f32(F32Args a) {
    __shared__ float hs[FT][FT + 1];
    __shared__ float ds[FT][FT + 1];
    poison_lds(hs, sizeof(hs));
    poison_lds(ds, sizeof(ds));
    const int n0 = blockIdx.x * FT;
    const int t0 = blockIdx.y * FT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t dF = (int64_t)a.d * a.F;
    const int64_t down_off = (a.swiglu ? 2 : 1) * dF;
    float y[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    for (int step = 0; step < a.P; ++step) {
        const int s = step;                              // records in ring order
        const float* wd = a.packed + (int64_t)s * a.shard_elems + down_off;   // F x d
        for (int k0 = 0; k0 < a.F; k0 += FT) {
            for (int i = threadIdx.x; i < FT * FT; i += 256) {
                const int r = i / FT, c = i % FT;
                const int tok = t0 + r, k = k0 + c;
                hs[r][c] = (tok < a.T && k < a.F) ? a.h[(int64_t)tok * a.f + (int64_t)s * a.F + k] : 0.f;
                const int kr = k0 + r, n = n0 + c;
                ds[r][c] = (kr < a.F && n < a.d) ? wd[(int64_t)kr * a.d + n] : 0.f;
            }
            __syncthreads();
            for (int k = 0; k < FT; ++k) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float hv = hs[ty * 2 + i][k];
#pragma unroll
                    for (int j = 0; j < 2; ++j) y[i][j] = fmaf(hv, ds[k][tx * 2 + j], y[i][j]);
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tok = t0 + ty * 2 + i;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + tx * 2 + j;
            if (tok < a.T && n < a.d) a.y[(int64_t)tok * a.d + n] = y[i][j];
        }
    }
}

hipError_t launch_gateup_f32(const F32Args& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.F + FT - 1) / FT), (unsigned)((a.T + FT - 1) / FT), (unsigned)a.P);
    if (a.swiglu)
        hipLaunchKernelGGL(gateup_f32<1>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(gateup_f32<2>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_down_f32(const F32Args& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.d + FT - 1) / FT), (unsigned)((a.T + FT - 1) / FT));
    hipLaunchKernelGGL(down_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace tsp
