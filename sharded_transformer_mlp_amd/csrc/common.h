// Device-side helpers shared by the gfx950 kernels of the sharded MLP path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsp {

#define TSP_LDS __attribute__((address_space(3)))

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void lgkm_zero() {
    __builtin_amdgcn_s_waitcnt((15 & 15) | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier that orders LDS traffic without draining the global
// loads still in flight for later stages (__syncthreads would wait for them).
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector: copies are plain loads and stores (HIP's uint4 is a
// struct whose copies can become memcpy and defeat register promotion).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The packed bf16 weight layout is built from 32 x 16 "fragment blocks":
// 32 output features (MFMA rows) by 16 reduction indices. A block is 512
// elements (1 KiB) stored in the order the 64 lanes of a wavefront consume
// them as the A operand of v_mfma_f32_32x32x16_bf16: lane l holds feature
// l % 32 and the 8 consecutive reduction indices 8 * (l / 32) .. + 7, so a
// wave reads one block with a single contiguous 16-byte-per-lane load. The
// token operand uses the same lane map (lane l: token l % 32). The 32 x 32
// fp32 result leaves lane l with token l % 32 and, in register 4 * q + r,
// feature 8 * q + 4 * (l / 32) + r (q, r = 0..3).
constexpr int FRAG_ELEMS = 512;

__host__ __device__ inline int64_t frag_offset(int64_t n, int64_t k, int64_t kblocks) {
    // element (feature n, reduction index k) in a matrix whose blocks run
    // k-fastest: block (n / 32, k / 16) is at ((n / 32) * kblocks + k / 16).
    return ((n >> 5) * kblocks + (k >> 4)) * FRAG_ELEMS + (((k & 15) >> 3) * 32 + (n & 31)) * 8 + (k & 7);
}

// SwiGLU packing interleaves gate and up in groups of 32 features: packed
// feature j of a shard is gate column 32 * (j / 64) + j % 32 when j % 64 < 32,
// and the up column of the same index otherwise. A 32-feature MFMA block is
// thus all-gate or all-up, and blocks 2q and 2q + 1 pair up element by element.

// Wavefront-uniform workgroup id remapped so that consecutive logical ids run
// on the same XCD: the dispatcher hands workgroup i to XCD i % 8, and tiles
// that share operands should share an L2.
__device__ inline int xcd_remap(int bid, int nwg) {
    const int q = nwg >> 3, r = nwg & 7;
    const int xcd = bid & 7, local = bid >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

// Token-tile-grouped raster over a (tokens x features) tile grid: GT token
// tiles share each feature tile, consecutive ids walk the token tiles first.
__device__ inline void raster(int L, int n_f, int n_t, int& ttile, int& flin, int GT = 8) {
    const int group = L / (GT * n_f);
    const int first = group * GT;
    const int gt = min(GT, n_t - first);
    const int rem = L - group * GT * n_f;
    ttile = first + rem % gt;
    flin = rem / gt;
}

// Both activations divide by 1 + e^x through the hardware reciprocal
// (v_rcp_f32, 1 ulp) instead of an IEEE division (about ten instructions):
// their results are rounded to bf16 or summed in fp32 right after, where one
// ulp is far below the path's error. e^x overflows to +inf for large x, and
// the reciprocal of +inf is 0, giving -0 for very negative inputs.
__device__ inline float silu_f(float g) {
    // g / (1 + e^-g)
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ inline float gelu_tanh_f(float u) {
    // 0.5 u (1 + tanh(z)) == u / (1 + e^{-2z}), z = sqrt(2/pi) (u + 0.044715 u^3)
    const float z2 = 1.5957691216057308f * (u + 0.044715f * u * u * u);
    return u * __builtin_amdgcn_rcpf(1.0f + __expf(-z2));
}

__device__ inline uint16_t bf16_bits(float x) {
    __bf16 b = static_cast<__bf16>(x);    // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

// fp16 (IEEE half) storage, round to nearest even; magnitudes above 65504
// become infinite.
__device__ inline uint16_t f16_bits(float x) {
    _Float16 h = static_cast<_Float16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ inline uint2 pack4_f16(float a, float b, float c, float d) {
    uint2 r;
    r.x = (uint32_t)f16_bits(a) | ((uint32_t)f16_bits(b) << 16);
    r.y = (uint32_t)f16_bits(c) | ((uint32_t)f16_bits(d) << 16);
    return r;
}

__device__ inline uint2 pack4_bf16(float a, float b, float c, float d) {
    uint2 r;
    r.x = (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
    r.y = (uint32_t)bf16_bits(c) | ((uint32_t)bf16_bits(d) << 16);
    return r;
}

// Debug builds (TSP_LDS_POISON) fill a kernel's LDS with NaN bit patterns
// (0x7FC0 in every 16-bit half: a bf16 NaN, and an fp32 NaN per word)
// before first use, so a fragment read that runs ahead of the data it waits
// for turns the output into NaN instead of reusing stale values.
__device__ inline void poison_lds(void* p, int bytes) {
#if TSP_LDS_POISON
    u32x4* q = static_cast<u32x4*>(p);
    const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    const int n = bytes / 16;
    const int nt = blockDim.x * blockDim.y * blockDim.z;
    for (int i = threadIdx.x; i < n; i += nt) q[i] = nan4;
    __syncthreads();
#else
    (void)p;
    (void)bytes;
#endif
}

}  // namespace tsp
