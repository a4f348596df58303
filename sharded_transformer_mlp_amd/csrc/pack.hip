// Shard packer: copies the caller's row-major weights into the library's
// per-shard records.
//
// Shard s of the block is the hidden-column range [s*F, (s+1)*F): those
// columns of the gate and up matrices and the same rows of the down matrix
// ("Tensor Parallelism: Splitting the Math", Megatron walk-through steps 2-5:
// column blocks of the first matrix, matching row blocks of the second).
// Each shard is one contiguous record, so a ring step would move one record.
// Records are stored in ring order: record k holds shard order[k], the shard
// a rank holds at ring step k. The forward kernels then walk records 0..P-1
// and never look the order up.
//
// bf16 record of shard s (all in 32 x 16 fragment blocks, see common.h):
//   [gate/up part]  NGU x d, NGU = 2F (SwiGLU, gate and up interleaved in
//                   groups of 32 features) or F (GeLU: columns of A);
//                   reduction index = model dim, d / 16 blocks per feature row.
//   [down part]     d x F: feature = output column n of the down matrix,
//                   reduction index = the shard's local hidden row, F / 16
//                   blocks per feature row.
#include "common.h"
#include "launch.h"

namespace tsp {

__global__ void pack_gateup_bf16(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                 uint16_t* __restrict__ dst, const int32_t* __restrict__ order,
                                 int64_t shard_elems, int d, int f, int F, int swiglu,
                                 int64_t chunks_per_shard) {
    const int64_t total = chunks_per_shard;
    const int rec = blockIdx.y;
    const int s = order[rec];
    const int kblocks = d >> 4;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = c >> 6;
        const int lane = (int)(c & 63);
        const int64_t nb = block / kblocks;
        const int kb = (int)(block - nb * kblocks);
        const int64_t j = nb * 32 + (lane & 31);          // packed feature within the shard
        const int k0 = kb * 16 + (lane >> 5) * 8;
        const uint16_t* src;
        int64_t col;
        if (swiglu) {
            src = ((j & 63) < 32) ? wg : wu;
            col = (int64_t)s * F + (j >> 6) * 32 + (j & 31);
        } else {
            src = wu;
            col = (int64_t)s * F + j;
        }
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[(int64_t)(k0 + e) * f + col];
        uint4 o;
        o.x = v[0] | ((uint32_t)v[1] << 16);
        o.y = v[2] | ((uint32_t)v[3] << 16);
        o.z = v[4] | ((uint32_t)v[5] << 16);
        o.w = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<uint4*>(dst + (int64_t)rec * shard_elems + c * 8) = o;
    }
}

__global__ void pack_down_bf16(const uint16_t* __restrict__ wd, uint16_t* __restrict__ dst,
                               const int32_t* __restrict__ order, int64_t shard_elems,
                               int64_t down_off, int d, int F, int64_t chunks_per_shard) {
    const int rec = blockIdx.y;
    const int s = order[rec];
    const int kblocks = F >> 4;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks_per_shard;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = c >> 6;
        const int lane = (int)(c & 63);
        const int64_t nb = block / kblocks;
        const int kb = (int)(block - nb * kblocks);
        const int64_t n = nb * 32 + (lane & 31);          // output feature (column of Wd)
        const int64_t r0 = (int64_t)s * F + kb * 16 + (lane >> 5) * 8;   // row of Wd
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = wd[(r0 + e) * d + n];
        uint4 o;
        o.x = v[0] | ((uint32_t)v[1] << 16);
        o.y = v[2] | ((uint32_t)v[3] << 16);
        o.z = v[4] | ((uint32_t)v[5] << 16);
        o.w = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<uint4*>(dst + (int64_t)rec * shard_elems + down_off + c * 8) = o;
    }
}

// The inverse of the two kernels above, for the backward: each 16-byte chunk
// of a record goes back to the 8 rows of its column it came from.
__global__ void unpack_gateup_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ wg,
                                   uint16_t* __restrict__ wu, const int32_t* __restrict__ order,
                                   int64_t shard_elems, int d, int f, int F, int swiglu,
                                   int64_t chunks_per_shard) {
    const int rec = blockIdx.y;
    const int s = order[rec];
    const int kblocks = d >> 4;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks_per_shard;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = c >> 6;
        const int lane = (int)(c & 63);
        const int64_t nb = block / kblocks;
        const int kb = (int)(block - nb * kblocks);
        const int64_t j = nb * 32 + (lane & 31);
        const int k0 = kb * 16 + (lane >> 5) * 8;
        uint16_t* dst;
        int64_t col;
        if (swiglu) {
            dst = ((j & 63) < 32) ? wg : wu;
            col = (int64_t)s * F + (j >> 6) * 32 + (j & 31);
        } else {
            dst = wu;
            col = (int64_t)s * F + j;
        }
        const uint4 o = *reinterpret_cast<const uint4*>(src + (int64_t)rec * shard_elems + c * 8);
        const uint32_t w4[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[(int64_t)(k0 + e) * f + col] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
}

__global__ void unpack_down_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ wd,
                                 const int32_t* __restrict__ order, int64_t shard_elems,
                                 int64_t down_off, int d, int F, int64_t chunks_per_shard) {
    const int rec = blockIdx.y;
    const int s = order[rec];
    const int kblocks = F >> 4;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks_per_shard;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = c >> 6;
        const int lane = (int)(c & 63);
        const int64_t nb = block / kblocks;
        const int kb = (int)(block - nb * kblocks);
        const int64_t n = nb * 32 + (lane & 31);
        const int64_t r0 = (int64_t)s * F + kb * 16 + (lane >> 5) * 8;
        const uint4 o = *reinterpret_cast<const uint4*>(src + (int64_t)rec * shard_elems + down_off + c * 8);
        const uint32_t w4[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) wd[(r0 + e) * d + n] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
}

// fp32 records keep the natural row-major orientation, per shard:
//   [gate cols d x F][up cols d x F][down rows F x d]  (GeLU: no gate part).
__global__ void pack_f32(const float* __restrict__ wg, const float* __restrict__ wu,
                         const float* __restrict__ wd, float* __restrict__ dst,
                         const int32_t* __restrict__ order, int64_t shard_elems, int d, int f,
                         int F, int swiglu) {
    const int rec = blockIdx.y;
    const int s = order[rec];
    const int64_t dF = (int64_t)d * F;
    const int64_t parts = swiglu ? 3 : 2;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < parts * dF;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t part = i / dF;
        const int64_t r = i - part * dF;
        float v;
        if (part < parts - 1) {                       // gate or up: d x F, row i, col c
            const int64_t row = r / F, col = r - row * F;
            const float* src = (swiglu && part == 0) ? wg : wu;
            v = src[row * f + (int64_t)s * F + col];
        } else {                                      // down: F x d
            const int64_t row = r / d, col = r - row * d;
            v = wd[((int64_t)s * F + row) * d + col];
        }
        dst[(int64_t)rec * shard_elems + i] = v;
    }
}

hipError_t launch_pack_bf16(const void* wg, const void* wu, const void* wd, void* dst,
                            const int32_t* order, int64_t shard_elems, int64_t down_off, int d,
                            int f, int F, int P, int swiglu, hipStream_t st) {
    const int64_t ngu = swiglu ? 2LL * F : (int64_t)F;
    const int64_t gu_chunks = ngu * d / 8, dn_chunks = (int64_t)d * F / 8;
    dim3 blk(256);
    dim3 g1((unsigned)std::min<int64_t>((gu_chunks + 255) / 256, 4096), P);
    hipLaunchKernelGGL(pack_gateup_bf16, g1, blk, 0, st, (const uint16_t*)wg,
                       (const uint16_t*)wu, (uint16_t*)dst, order, shard_elems, d, f, F, swiglu,
                       gu_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2((unsigned)std::min<int64_t>((dn_chunks + 255) / 256, 4096), P);
    hipLaunchKernelGGL(pack_down_bf16, g2, blk, 0, st, (const uint16_t*)wd, (uint16_t*)dst, order,
                       shard_elems, down_off, d, F, dn_chunks);
    return hipGetLastError();
}

// Row-major M x K (row stride ld) into 32 x 16 fragment blocks, the layout
// of the packed records (block (m / 32, k / 16) at ((m / 32) (K / 16) + k / 16)
// 512, lane l holding row l % 32 and indices 8 (l / 32) .. + 7): one 16-byte
// lane slot per thread. The backward's dX product reads Wg and Wu so.
__global__ void pack_frag_bf16(const uint16_t* __restrict__ src, int64_t ld, int K, uint16_t* __restrict__ dst,
                               int64_t chunks) {
    const int kb_per_row = K >> 4;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = c >> 6;
        const int lane = (int)(c & 63);
        const int64_t nb = block / kb_per_row;
        const int kb = (int)(block - nb * kb_per_row);
        const int64_t row = nb * 32 + (lane & 31);
        const int k0 = kb * 16 + (lane >> 5) * 8;
        *reinterpret_cast<u32x4*>(dst + c * 8) = *reinterpret_cast<const u32x4*>(src + row * ld + k0);
    }
}

hipError_t launch_pack_frag_bf16(const uint16_t* src, int64_t ld, int M, int K, uint16_t* dst, hipStream_t st) {
    if (M % 32 || K % 16 || ld % 8 || ld < K) return hipErrorInvalidValue;
    const int64_t chunks = (int64_t)M * K / 8;
    const dim3 grid((unsigned)std::min<int64_t>((chunks + 255) / 256, 8192));
    hipLaunchKernelGGL(pack_frag_bf16, grid, dim3(256), 0, st, src, ld, K, dst, chunks);
    return hipGetLastError();
}

hipError_t launch_unpack_bf16(const void* src, void* wg, void* wu, void* wd, const int32_t* order,
                              int64_t shard_elems, int64_t down_off, int d, int f, int F, int P, int swiglu,
                              hipStream_t st) {
    const int64_t ngu = swiglu ? 2LL * F : (int64_t)F;
    const int64_t gu_chunks = ngu * d / 8, dn_chunks = (int64_t)d * F / 8;
    dim3 blk(256);
    dim3 g1((unsigned)std::min<int64_t>((gu_chunks + 255) / 256, 4096), P);
    hipLaunchKernelGGL(unpack_gateup_bf16, g1, blk, 0, st, (const uint16_t*)src, (uint16_t*)wg, (uint16_t*)wu,
                       order, shard_elems, d, f, F, swiglu, gu_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2((unsigned)std::min<int64_t>((dn_chunks + 255) / 256, 4096), P);
    hipLaunchKernelGGL(unpack_down_bf16, g2, blk, 0, st, (const uint16_t*)src, (uint16_t*)wd, order, shard_elems,
                       down_off, d, F, dn_chunks);
    return hipGetLastError();
}

hipError_t launch_pack_f32(const void* wg, const void* wu, const void* wd, void* dst,
                           const int32_t* order, int64_t shard_elems, int d, int f, int F, int P,
                           int swiglu, hipStream_t st) {
    const int64_t n = (swiglu ? 3 : 2) * (int64_t)d * F;
    dim3 g((unsigned)std::min<int64_t>((n + 255) / 256, 4096), P);
    hipLaunchKernelGGL(pack_f32, g, dim3(256), 0, st, (const float*)wg, (const float*)wu,
                       (const float*)wd, (float*)dst, order, shard_elems, d, f, F, swiglu);
    return hipGetLastError();
}

}  // namespace tsp

namespace tsp {

// Row shards of one (P F) x d matrix, F rows per shard, packed like the down
// part of an MLP record with no gate/up part before it (the attention
// block's output projection).
hipError_t launch_pack_rows_bf16(const void* w, void* dst, const int32_t* order, int64_t rec_elems, int d,
                                 int F, int P, hipStream_t st) {
    const int64_t chunks = (int64_t)d * F / 8;
    dim3 g((unsigned)std::min<int64_t>((chunks + 255) / 256, 4096), P);
    hipLaunchKernelGGL(pack_down_bf16, g, dim3(256), 0, st, (const uint16_t*)w, (uint16_t*)dst, order, rec_elems,
                       (int64_t)0, d, F, chunks);
    return hipGetLastError();
}

}  // namespace tsp
