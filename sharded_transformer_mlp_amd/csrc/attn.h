// Internal launchers of the attention block (C++ linkage, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsp {

// Head dimension the attention kernels are written for.
constexpr int ATT_DH = 128;

// Q/K/V projection of a rank's T tokens over all P head-group records.
struct ProjArgs {
    const uint16_t* packed;   // P records of d x Fqkv, Fqkv = (Hs + 2 Hks) * 128, visiting order
    const uint16_t* x;        // T x d tokens
    uint16_t* q;              // T x ldq queries (scaled by q_scale); group at visiting step k: columns [k Hs 128, (k+1) Hs 128)
    uint16_t* kc;             // key context, rows = sequence positions, ld = ldk, key/value head j at j * 128
    uint16_t* vt;             // value context transposed: row j * 128 + c, sequence positions along the row
    const int32_t* order;     // visiting step -> head group (device)
    int64_t rec_elems, ldq, ldk, ldv, row0;   // row0: sequence position of token 0 (rank * T)
    int T, d, P, Hs, Hks;
    float q_scale;            // queries are stored times this (log2(e) / sqrt(128)), rounded once
};

// Causal (or full) attention of a rank's queries over the context.
struct AttnArgs {
    const uint16_t* q;        // as ProjArgs::q
    const uint16_t* kc;
    const uint16_t* vt;
    uint16_t* o;              // T x ldq, same layout as q
    const int32_t* order;
    int64_t ldq, ldk, ldv;
    int T, S, row0, P, Hs, Hks, causal;
    int hw, qs, n_qt, n_hq;   // heads per workgroup, 64-query sub-tiles per workgroup, query tiles, head quarters
    float scale_log2;         // log2(e) / sqrt(128), the scale the projection applied to the queries
};

hipError_t launch_pack_qkv_bf16(const void* wq, const void* wk, const void* wv, void* dst, const int32_t* order,
                                int64_t rec_elems, int d, int H, int Hkv, int dh, int P, hipStream_t st);
hipError_t launch_pack_rows_bf16(const void* w, void* dst, const int32_t* order, int64_t rec_elems, int d,
                                 int F, int P, hipStream_t st);
hipError_t launch_qkv(const ProjArgs& a, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

}  // namespace tsp
