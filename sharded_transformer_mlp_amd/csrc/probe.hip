// Ceiling probes: what this GPU sustains on the two resources the MLP block
// is bound by, for reporting the block's kernels against measured ceilings
// beside the datasheet peaks. Not on the forward path.
//
// probe_hbm_read: a grid-stride stream of 16-byte nontemporal loads (the
//   load form the weight-streaming kernels use) over a buffer larger than
//   every cache, folded with XOR so the loads cannot be dropped.
// probe_mfma_bf16: every wave keeps 16 independent 16 x 16 fp32 accumulators
//   and issues v_mfma_f32_16x16x32_bf16 back to back on pseudo-random bf16
//   operands spread like unit-variance data (random sign and mantissa,
//   exponents 2^-1 .. 2^2), two waves per SIMD.
#include "common.h"
#include "launch.h"

namespace tsp {

constexpr int PROBE_HBM_THREADS = 256, PROBE_HBM_U = 4;

__global__ __launch_bounds__(PROBE_HBM_THREADS) void probe_hbm_read(const u32x4* __restrict__ src, int64_t n,
                                                                     u32x4* __restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * PROBE_HBM_THREADS * PROBE_HBM_U;
    for (int64_t base = (int64_t)blockIdx.x * PROBE_HBM_THREADS * PROBE_HBM_U + threadIdx.x; base < n;
         base += stride) {
        u32x4 v[PROBE_HBM_U];
#pragma unroll
        for (int u = 0; u < PROBE_HBM_U; ++u) {
            const int64_t i = base + (int64_t)u * PROBE_HBM_THREADS;
            v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < PROBE_HBM_U; ++u) acc ^= v[u];
    }
    // the buffer is zero-filled, so this store never happens; the compiler
    // cannot know that and keeps every load
    if ((acc.x | acc.y | acc.z | acc.w) != 0u) sink[0] = acc;
}

__device__ inline bf16x8 probe_operand(uint32_t seed) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        seed = seed * 1664525u + 1013904223u;
        const uint32_t lo = (seed & 0x807fu) | ((126u + ((seed >> 8) & 3u)) << 7);
        const uint32_t hi = ((seed >> 16) & 0x807fu) | ((126u + ((seed >> 24) & 3u)) << 7);
        v[e] = lo | (hi << 16);
    }
    return __builtin_bit_cast(bf16x8, v);
}

constexpr int PROBE_MFMA_THREADS = 512;

__global__ __launch_bounds__(PROBE_MFMA_THREADS) void probe_mfma_bf16(int iters, float* __restrict__ sink) {
    const uint32_t tid = blockIdx.x * PROBE_MFMA_THREADS + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = probe_operand(tid * 2654435761u + 97u * i);
        b[i] = probe_operand(tid * 40503u + 131u * i + 7u);
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    sink[tid] = s;
}

hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, void* sink, hipStream_t st) {
    const int64_t n = bytes / 16;
    hipLaunchKernelGGL(probe_hbm_read, dim3(4096), dim3(PROBE_HBM_THREADS), 0, st,
                       static_cast<const u32x4*>(buf), n, static_cast<u32x4*>(sink));
    return hipGetLastError();
}

int probe_mfma_blocks() { return 256 * 4; }       // 4 workgroups of 8 waves per CU: 8 waves per SIMD over time
int probe_mfma_threads() { return PROBE_MFMA_THREADS; }
double probe_mfma_flops(int iters) {
    return (double)probe_mfma_blocks() * (PROBE_MFMA_THREADS / 64) * iters * 16 * (2.0 * 16 * 16 * 32);
}

hipError_t launch_probe_mfma_bf16(int iters, float* sink, hipStream_t st) {
    hipLaunchKernelGGL(probe_mfma_bf16, dim3(probe_mfma_blocks()), dim3(PROBE_MFMA_THREADS), 0, st, iters, sink);
    return hipGetLastError();
}

}  // namespace tsp
