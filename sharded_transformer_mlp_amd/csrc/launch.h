// Internal launchers (C++ linkage, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace tsp {

// Per-forward description shared by the bf16 kernels.
struct Bf16Args {
    const uint16_t* packed;   // packed weights (all shard records)
    const uint16_t* x;        // T x d tokens
    uint16_t* h;              // T x f hidden activations (workspace), columns in ring-step order
    float* y;                 // T x d output
    float* part;              // split-reduction partials, split x T x d fp32 (workspace; may be null)
    int64_t shard_elems;      // elements per shard record (records in ring order)
    int64_t down_off;         // offset of the down part inside a record
    int T, d, f, F, P;
    int swiglu;
};

struct F32Args {
    const float* packed;
    const float* x;
    float* h;
    float* y;
    int64_t shard_elems;
    int T, d, f, F, P;
    int swiglu;
};

// Pack the weights into P records in ring order (record k = shard order[k]).
hipError_t launch_pack_bf16(const void* wg, const void* wu, const void* wd, void* dst,
                            const int32_t* order, int64_t shard_elems, int64_t down_off, int d,
                            int f, int F, int P, int swiglu, hipStream_t st);
hipError_t launch_pack_f32(const void* wg, const void* wu, const void* wd, void* dst,
                           const int32_t* order, int64_t shard_elems, int d, int f, int F, int P,
                           int swiglu, hipStream_t st);

// Tiled MFMA path. Each returns the launch status; `cfg` picks a tile shape.
hipError_t launch_gateup_tiled(const Bf16Args& a, int cfg, hipStream_t st);
// split > 1 (shape 5 only): the ring is cut into `split` groups of
// consecutive ring steps, each group's sum goes to its own fp32 partial in
// a.part, and launch_reduce_partials adds the partials in ring order into Y.
hipError_t launch_down_tiled(const Bf16Args& a, int cfg, int split, hipStream_t st);
hipError_t launch_reduce_partials(const float* part, int split, int64_t n, float* y, hipStream_t st);
// Number of ring-step groups for the down product at this shape (1 = none).
int choose_down_split(int T, int d, int P, int cfg);
// Bytes of partials the largest split needs for any T <= T_max.
int64_t down_split_bytes(int64_t T_max, int d, int P);
// Tile-shape choice for a shape (host logic; -1 = none fits).
int choose_gateup_cfg(int T, int d, int F, int P, int swiglu);
int choose_down_cfg(int T, int d, int F, int P);
const char* tiled_cfg_name(int cfg);
bool gateup_cfg_fits(int cfg, int d, int F, int swiglu);
bool down_cfg_fits(int cfg, int d, int F);

// Skinny weight-streaming path (T <= SKINNY_T_MAX).
constexpr int SKINNY_T_MAX = 48;
hipError_t launch_gateup_skinny(const Bf16Args& a, hipStream_t st);
hipError_t launch_down_skinny(const Bf16Args& a, hipStream_t st);
bool skinny_supported(int d, int F, int P);

// Backward (bf16). C[n][m] = sum_k A[m][k] B[n][k] over nseg segments of spp
// 32-deep steps; segment j reads A at a_base[j % kinds] + (order ? order[j /
// kinds] : j / kinds) * a_seg and B at b_base[j % kinds] + (j / kinds) * b_seg.
// Output fp32 out[row(n) * ldc + col(m)] for n < N; remap 1 / 2 maps the
// column / row index from ring order to the shard's natural position
// (remap_order, shard width F).
struct NtArgs {
    const uint16_t* a_base[2];
    const uint16_t* b_base[2];
    int64_t a_seg, b_seg;
    const int32_t* order;
    int lda, ldb, M, N, spp, nseg, kinds;
    float* out;
    int64_t ldc;
    int remap, F;
    const int32_t* remap_order;
};
struct BwdArgs {
    const float* dh;          // T x f fp32, natural hidden columns
    uint16_t* dg;             // T x f bf16, ring-ordered hidden columns (SwiGLU only)
    uint16_t* du;             // T x f bf16, ring-ordered
    uint16_t* h;              // T x f bf16, ring-ordered
    const int32_t* order;     // ring order (device)
};
hipError_t launch_transpose_bf16(const uint16_t* src, int R, int C, int ld_src, uint16_t* dst, int R_pad,
                                 hipStream_t st);
// Up to three products in one launch; first[i] is product i's first tile.
struct NtGroup {
    NtArgs p[3];
    int first[3];
};
hipError_t launch_nt(const NtArgs* probs, int n, hipStream_t st);
hipError_t launch_gateup_bwd(const Bf16Args& a, const BwdArgs& b, hipStream_t st);

// fp32 path.
hipError_t launch_gateup_f32(const F32Args& a, hipStream_t st);
hipError_t launch_down_f32(const F32Args& a, hipStream_t st);

// Ceiling probes (measurement only).
hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, void* sink, hipStream_t st);
hipError_t launch_probe_mfma_bf16(int iters, float* sink, hipStream_t st);
int probe_mfma_blocks();
int probe_mfma_threads();
double probe_mfma_flops(int iters);

}  // namespace tsp
