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
    // H in 16-token x 32-column blocks (1 KiB, row-major inside), block
    // (column block kb, token block tb) at (kb * nbt + tb) * 512 elements, with
    // nbt = ceil(T / 16); 0 = H row-major T x f. Only the 256 x 256 kernels
    // (tile shape 0 for both products) take the blocked layout.
    int nbt = 0;
    // Tile shape 0 gate/up only, may be null: every tile's accumulators (the
    // gate and up pre-activations, fp32) in the saved-activation layout (see
    // w16::save_acc), gateup_saved_bytes(T, F, P, swiglu) bytes.
    float* save = nullptr;
    // Token tiles per raster group of the tile shape 0 kernels (set from the
    // shape by launch_gateup_tiled and launch_down_tiled)
    int gt = 8;
};

struct F32Args {
    const float* packed;
    const float* x;
    float* h;
    float* y;
    float* part;              // split > 1: split fp32 partials of T x d
    int64_t shard_elems;
    int T, d, f, F, P;
    int swiglu;
    int split = 1;            // reduction groups of the down product (choose_f32_split)
};

// Pack the weights into P records in ring order (record k = shard order[k]).
hipError_t launch_pack_bf16(const void* wg, const void* wu, const void* wd, void* dst,
                            const int32_t* order, int64_t shard_elems, int64_t down_off, int d,
                            int f, int F, int P, int swiglu, hipStream_t st);
// Inverse of launch_pack_bf16: the records back into row-major wg, wu (d x f)
// and wd (f x d), bit for bit (wg unused for GeLU).
hipError_t launch_unpack_bf16(const void* src, void* wg, void* wu, void* wd, const int32_t* order,
                              int64_t shard_elems, int64_t down_off, int d, int f, int F, int P, int swiglu,
                              hipStream_t st);
hipError_t launch_pack_f32(const void* wg, const void* wu, const void* wd, void* dst,
                           const int32_t* order, int64_t shard_elems, int d, int f, int F, int P,
                           int swiglu, hipStream_t st);

// Tiled MFMA path. Each returns the launch status; `cfg` picks a tile shape.
hipError_t launch_gateup_tiled(const Bf16Args& a, int cfg, hipStream_t st);
// split > 1 (tile shape 0 only): the ring is cut into `split` groups of
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
// (remap_order, shard width F). a_frag: A is stored in 32 x 16 fragment
// blocks with K = lda (see RowSrc in w16.h), the same for every product of
// one launch.
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
    int a_frag;
};
struct BwdArgs {
    const float* dh;          // T x f fp32, natural hidden columns
    uint16_t* dg;             // T x f bf16, ring-ordered hidden columns (SwiGLU only)
    uint16_t* du;             // T x f bf16, ring-ordered
    uint16_t* dgt;            // the same transposed (f rows x ldt tokens) in 32 x 16 fragment blocks (SwiGLU only)
    uint16_t* dut;            // f x ldt, fragment blocks
    uint16_t* ht;             // H transposed, f x ldt row-major, tokens contiguous
    int ldt;                  // T rounded up to 64; columns T..ldt-1 hold finite values
    const int32_t* order;     // ring order (device)
    // null: recompute the gate/up product; else the accumulators a forward
    // saved (Bf16Args::save) for the same weights, T and X
    const float* saved = nullptr;
};
// dst[c][r] = src[r][c] (R x C bf16 source, row stride ld_src) for r < R,
// 0 for R <= r < R_pad; frag: dst in 32 x 16 fragment blocks (C rows x R_pad
// reduction indices) instead of row-major C x R_pad. C % 64 == 0, R_pad % 64
// == 0. Runs as extra workgroups of a grouped NT launch (launch_nt).
struct TransposeJob {
    const uint16_t* src;
    uint16_t* dst;
    int R, C, ld_src, R_pad, frag;
};
constexpr int kMaxTp = 2;
// Row-major M x K (row stride ld) into 32 x 16 fragment blocks (M % 32 == 0,
// K % 16 == 0, ld % 8 == 0).
hipError_t launch_pack_frag_bf16(const uint16_t* src, int64_t ld, int M, int K, uint16_t* dst, hipStream_t st);
// Up to four products in one launch; first[i] is product i's first tile.
constexpr int kMaxNt = 4;
// Transposes (up to kMaxTp) may ride along: workgroup ids from aux_first on
// each walk the jobs' 64 x 64 tiles, n_aux apart. They come after every
// product tile, so they take the CUs that the products' last partial round
// leaves idle.
struct NtGroup {
    NtArgs p[kMaxNt];
    int first[kMaxNt];
    TransposeJob tp[kMaxTp];
    int n_tp, aux_first, n_aux;
};
hipError_t launch_nt(const NtArgs* probs, int n, hipStream_t st, const TransposeJob* tps = nullptr, int n_tp = 0);
hipError_t launch_gateup_bwd(const Bf16Args& a, const BwdArgs& b, hipStream_t st);
// Bytes of the saved gate/up accumulators for T tokens: one 256 KiB tile per
// (256-token tile, 256-row block of a shard's packed gate/up rows).
int64_t gateup_saved_bytes(int64_t T, int64_t F, int P, int swiglu);

// fp32 path.
hipError_t launch_gateup_f32(const F32Args& a, hipStream_t st);
hipError_t launch_down_f32(const F32Args& a, hipStream_t st);
hipError_t launch_reduce_f32(const float* part, int split, int64_t n, float* y, hipStream_t st);
// Reduction groups of the fp32 down product at this shape (1 = none), and the
// partials' bytes the largest split needs for any T <= T_max.
int choose_f32_split(int T, int d, int F);
int64_t f32_split_bytes(int64_t T_max, int d, int F);

// Ceiling probes (measurement only).
hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, void* sink, hipStream_t st);
hipError_t launch_probe_mfma_bf16(int iters, float* sink, hipStream_t st);
int probe_mfma_blocks();
int probe_mfma_threads();
double probe_mfma_flops(int iters);

}  // namespace tsp
