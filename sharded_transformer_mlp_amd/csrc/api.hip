// C ABI of the sharded gated-MLP hot path: argument checks, the per-handle
// packed weights and workspace, and the per-forward launch plan.
#include "tsp_mlp.h"
#include "tsp_attn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "attn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

tsp_status_t fail(tsp_status_t s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

tsp_status_t hip_fail(hipError_t e, const char* what) {
    return fail(TSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int kMaxTimingPairs = 8192;

struct KernelTotal {
    std::string name;
    double ms = 0.0;
    int64_t launches = 0;
};

struct EventPair {
    hipEvent_t start = nullptr, stop = nullptr;
    int slot = 0;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct tsp_mlp {
    int64_t T_max = 0, d = 0, f = 0, F = 0;
    int32_t P = 0, act = 0, dtype = 0;
    std::vector<int32_t> order;
    int device = 0;
    hipStream_t stream = nullptr;
    int32_t* order_dev = nullptr;
    void* packed = nullptr;
    int64_t packed_bytes = 0, shard_elems = 0, down_off = 0;
    void* work = nullptr;
    int64_t work_bytes = 0;
    void* bwd = nullptr;                       // backward workspace (first backward call)
    int64_t bwd_bytes = 0;
    bool bwd_unpacked = false;                 // the weights in the backward workspace are filled
    int64_t part_off = 0;                      // byte offset of the down-split partials in work
    int32_t path = TSP_PATH_AUTO;
    int32_t cfg_gateup = -1, cfg_down = -1;   // tiled shapes; -1 = chosen per forward
    // kernel timing
    bool timing = false;
    std::vector<EventPair> pool;
    size_t used = 0;
    std::vector<KernelTotal> totals;
};

namespace {

int timing_slot(tsp_mlp* h, const char* name) {
    for (size_t i = 0; i < h->totals.size(); ++i)
        if (h->totals[i].name == name) return (int)i;
    h->totals.push_back(KernelTotal{name, 0.0, 0});
    return (int)h->totals.size() - 1;
}

tsp_status_t drain_timing(tsp_mlp* h) {
    for (size_t i = 0; i < h->used; ++i) {
        EventPair& e = h->pool[i];
        hipError_t err = hipEventSynchronize(e.stop);
        if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
        float ms = 0.f;
        err = hipEventElapsedTime(&ms, e.start, e.stop);
        if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
        h->totals[e.slot].ms += ms;
        h->totals[e.slot].launches += 1;
    }
    h->used = 0;
    return TSP_OK;
}

// Runs `launch` on `st`, bracketed by events when timing is on.
template <class Fn>
tsp_status_t timed_launch(tsp_mlp* h, const char* name, hipStream_t st, Fn&& launch) {
    EventPair* ep = nullptr;
    if (h->timing) {
        if (h->used == h->pool.size()) {
            if (h->pool.size() < (size_t)kMaxTimingPairs) {
                // timing-only events: no system-scope fence (its cache
                // writeback and invalidation would slow the next kernel)
                EventPair e;
                hipError_t err = hipEventCreateWithFlags(&e.start, hipEventDisableSystemFence);
                if (err == hipSuccess) err = hipEventCreateWithFlags(&e.stop, hipEventDisableSystemFence);
                if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
                h->pool.push_back(e);
            } else {
                tsp_status_t s = drain_timing(h);   // pool full: fold the finished pairs in
                if (s != TSP_OK) return s;
            }
        }
        ep = &h->pool[h->used++];
        ep->slot = timing_slot(h, name);
        hipError_t err = hipEventRecord(ep->start, st);
        if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    }
    hipError_t err = launch();
    if (err != hipSuccess) return fail(TSP_ERR_HIP, "launch of %s: %s", name, hipGetErrorString(err));
    if (ep) {
        err = hipEventRecord(ep->stop, st);
        if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    }
    return TSP_OK;
}

void free_buffers(tsp_mlp* h) {
    for (EventPair& e : h->pool) {
        if (e.start) (void)hipEventDestroy(e.start);
        if (e.stop) (void)hipEventDestroy(e.stop);
    }
    h->pool.clear();
    if (h->order_dev) (void)hipFree(h->order_dev);
    if (h->packed) (void)hipFree(h->packed);
    if (h->work) (void)hipFree(h->work);
    if (h->bwd) (void)hipFree(h->bwd);
    h->order_dev = nullptr;
    h->packed = h->work = h->bwd = nullptr;
}

void release(tsp_mlp* h) {
    if (!h) return;
    free_buffers(h);
    delete h;
}

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

}  // namespace

extern "C" {

const char* tsp_status_string(tsp_status_t s) {
    switch (s) {
        case TSP_OK: return "ok";
        case TSP_ERR_INVALID_ARG: return "invalid argument";
        case TSP_ERR_UNSUPPORTED: return "unsupported shape";
        case TSP_ERR_OOM: return "out of device memory";
        case TSP_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* tsp_last_error(void) { return g_last_error.c_str(); }

tsp_status_t tsp_mlp_validate(int64_t T_max, int64_t d, int64_t f, int32_t P, int32_t act,
                              int32_t dtype, const int32_t* order, int32_t has_gate) {
    if (T_max < 1 || T_max > kMaxDim) return fail(TSP_ERR_INVALID_ARG, "T_max=%lld out of [1, 2^30]", (long long)T_max);
    if (d < 1 || d > kMaxDim) return fail(TSP_ERR_INVALID_ARG, "d=%lld out of [1, 2^30]", (long long)d);
    if (f < 1 || f > kMaxDim) return fail(TSP_ERR_INVALID_ARG, "f=%lld out of [1, 2^30]", (long long)f);
    if (P < 1 || P > f) return fail(TSP_ERR_INVALID_ARG, "P=%d out of [1, f]", P);
    if (f % P) return fail(TSP_ERR_INVALID_ARG, "P=%d does not divide f=%lld", P, (long long)f);
    if (act != TSP_ACT_SWIGLU && act != TSP_ACT_GELU_TANH) return fail(TSP_ERR_INVALID_ARG, "unknown activation %d", act);
    if (dtype != TSP_DTYPE_F32 && dtype != TSP_DTYPE_BF16) return fail(TSP_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if ((has_gate != 0) != (act == TSP_ACT_SWIGLU))
        return fail(TSP_ERR_INVALID_ARG, act == TSP_ACT_SWIGLU ? "SwiGLU needs a gate matrix" : "GeLU takes no gate matrix");
    if (order) {
        std::vector<char> seen((size_t)P, 0);
        for (int32_t k = 0; k < P; ++k) {
            const int32_t s = order[k];
            if (s < 0 || s >= P || seen[(size_t)s]) return fail(TSP_ERR_INVALID_ARG, "order is not a permutation of 0..P-1 (entry %d = %d)", k, s);
            seen[(size_t)s] = 1;
        }
    }
    const int64_t F = f / P;
    if (dtype == TSP_DTYPE_BF16 && (d % 64 || F % 64))
        return fail(TSP_ERR_UNSUPPORTED, "bf16 path needs d and F = f/P to be multiples of 64 (d=%lld, F=%lld)", (long long)d, (long long)F);
    const int64_t es = dtype == TSP_DTYPE_BF16 ? 2 : 4;
    if (T_max * f > (int64_t(1) << 40) / es)      // workspace bound keeps every index in range
        return fail(TSP_ERR_UNSUPPORTED, "T_max * f too large");
    return TSP_OK;
}

tsp_status_t tsp_mlp_create(tsp_mlp_t* out, int64_t T_max, int64_t d, int64_t f, int32_t P,
                            int32_t act, int32_t dtype, const int32_t* order, const void* w_gate,
                            const void* w_up, const void* w_down, hipStream_t stream) {
    if (!out) return fail(TSP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    tsp_status_t s = tsp_mlp_validate(T_max, d, f, P, act, dtype, order, w_gate != nullptr);
    if (s != TSP_OK) return s;
    if (!w_up || !w_down) return fail(TSP_ERR_INVALID_ARG, "weight pointer is NULL");
    if (!aligned16(w_up) || !aligned16(w_down) || (w_gate && !aligned16(w_gate)))
        return fail(TSP_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");

    tsp_mlp* h = new (std::nothrow) tsp_mlp;
    if (!h) return fail(TSP_ERR_OOM, "host allocation failed");
    h->T_max = T_max; h->d = d; h->f = f; h->P = P; h->F = f / P;
    h->act = act; h->dtype = dtype; h->stream = stream;
    h->order.resize((size_t)P);
    for (int32_t k = 0; k < P; ++k) h->order[(size_t)k] = order ? order[k] : k;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) { release(h); return hip_fail(e, "hipGetDevice"); }

    const bool swiglu = act == TSP_ACT_SWIGLU;
    const int64_t F = h->F;
    int64_t es;
    if (dtype == TSP_DTYPE_BF16) {
        const int64_t ngu = swiglu ? 2 * F : F;
        h->down_off = ngu * d;
        h->shard_elems = ngu * d + d * F;
        es = 2;
    } else {
        h->down_off = (swiglu ? 2 : 1) * d * F;
        h->shard_elems = (swiglu ? 3 : 2) * d * F;
        es = 4;
    }
    h->packed_bytes = h->shard_elems * P * es;
    // workspace: hidden activations (tiled and fp32 paths: T_max x f; skinny:
    // f / 16 fragment blocks of 1 KiB per 32-token block; the larger of the
    // two), then for bf16 the fp32 partials of a ring-group split of the down
    // product (at most 64 MiB, see down_split_bytes)
    h->work_bytes = (T_max + 15) / 16 * 16 * f * es;     // whole 16-token blocks of H
    if (dtype == TSP_DTYPE_BF16) {
        const int64_t ntb = ((T_max < tsp::SKINNY_T_MAX ? T_max : tsp::SKINNY_T_MAX) + 31) / 32;
        if (ntb * 32 * f * 2 > h->work_bytes) h->work_bytes = ntb * 32 * f * 2;
    }
    h->work_bytes = (h->work_bytes + 255) / 256 * 256;
    h->part_off = h->work_bytes;
    if (dtype == TSP_DTYPE_BF16) h->work_bytes += tsp::down_split_bytes(T_max, (int)d, P);
    else h->work_bytes += tsp::f32_split_bytes(T_max, (int)d, (int)h->F);

    if ((e = hipMalloc(&h->order_dev, sizeof(int32_t) * (size_t)P)) != hipSuccess ||
        (e = hipMalloc(&h->packed, (size_t)h->packed_bytes)) != hipSuccess ||
        (e = hipMalloc(&h->work, (size_t)h->work_bytes)) != hipSuccess) {
        const bool oom = e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation;
        release(h);
        (void)hipGetLastError();
        return oom ? fail(TSP_ERR_OOM, "device allocation of packed weights / workspace failed")
                   : hip_fail(e, "hipMalloc");
    }
    e = hipMemcpyAsync(h->order_dev, h->order.data(), sizeof(int32_t) * (size_t)P, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) { release(h); return hip_fail(e, "hipMemcpyAsync(order)"); }
    if (dtype == TSP_DTYPE_BF16)
        e = tsp::launch_pack_bf16(w_gate, w_up, w_down, h->packed, h->order_dev, h->shard_elems,
                                  h->down_off, (int)d, (int)f, (int)F, P, swiglu ? 1 : 0, stream);
    else
        e = tsp::launch_pack_f32(w_gate, w_up, w_down, h->packed, h->order_dev, h->shard_elems,
                                 (int)d, (int)f, (int)F, P, swiglu ? 1 : 0, stream);
    if (e != hipSuccess) { release(h); return hip_fail(e, "pack launch"); }
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) { release(h); return hip_fail(e, "hipStreamSynchronize after packing"); }
    *out = h;
    return TSP_OK;
}

}  // extern "C"

namespace {

// Workspace bytes a forward of T tokens needs (the hidden activations, then
// the down-split partials at part_off), for the path and tile shapes the
// forward will take.
struct FwdPlan {
    bool skinny = false;
    int cg = -1, cd = -1, split = 1, nbt = 0;
    int64_t h_bytes = 0, part_off = 0, total = 0;
};

// train: the forward that saves the gate/up pre-activations, which only the
// tiled gate/up kernel of shape 0 does (whatever the path and tile settings).
tsp_status_t plan_forward(const tsp_mlp* h, int64_t T, FwdPlan& pl, bool train = false) {
    const int64_t d = h->d, f = h->f;
    if (h->dtype == TSP_DTYPE_BF16) {
        const bool sk_ok = T <= tsp::SKINNY_T_MAX && tsp::skinny_supported((int)d, (int)h->F, h->P);
        if (train) {
            pl.skinny = false;
        } else if (h->path == TSP_PATH_SKINNY) {
            if (!sk_ok) return fail(TSP_ERR_UNSUPPORTED, "skinny path needs T <= %d, d %% 256 == 0 and P*F %% 1024 == 0", tsp::SKINNY_T_MAX);
            pl.skinny = true;
        } else if (h->path == TSP_PATH_AUTO) {
            pl.skinny = sk_ok;
        }
        if (pl.skinny) {
            pl.h_bytes = (T + 31) / 32 * 32 * f * 2;
        } else {
            const int swiglu = h->act == TSP_ACT_SWIGLU ? 1 : 0;
            pl.cg = train ? 0 : h->cfg_gateup >= 0 ? h->cfg_gateup : tsp::choose_gateup_cfg((int)T, (int)d, (int)h->F, h->P, swiglu);
            pl.cd = h->cfg_down >= 0 ? h->cfg_down : tsp::choose_down_cfg((int)T, (int)d, (int)h->F, h->P);
            if (pl.cg < 0 || pl.cd < 0) return fail(TSP_ERR_UNSUPPORTED, "no tile shape fits d=%lld F=%lld", (long long)d, (long long)h->F);
            pl.split = tsp::choose_down_split((int)T, (int)d, h->P, pl.cd);
            const int64_t n_tok_tiles = (T + 63) / 64;
            if (n_tok_tiles * (2 * f / 64 + d / 64) > INT32_MAX / 2) return fail(TSP_ERR_UNSUPPORTED, "grid too large");
            // blocked H (both products on the 256 x 256 kernels) fills whole
            // 16-token blocks
            pl.nbt = (pl.cg == 0 && pl.cd == 0) ? (int)((T + 15) / 16) : 0;
            pl.h_bytes = (T + 15) / 16 * 16 * f * 2;
        }
    } else {
        if (h->path == TSP_PATH_SKINNY) return fail(TSP_ERR_UNSUPPORTED, "skinny path is bf16 only");
        pl.h_bytes = T * f * 4;
        pl.split = tsp::choose_f32_split((int)T, (int)d, (int)h->F);
    }
    pl.part_off = (pl.h_bytes + 255) / 256 * 256;
    pl.total = pl.part_off + (pl.split > 1 ? (int64_t)pl.split * T * d * 4 : 0);
    return TSP_OK;
}

tsp_status_t check_forward_args(const tsp_mlp* h, int64_t T, const void* X, const float* Y) {
    if (!X || !Y) return fail(TSP_ERR_INVALID_ARG, "X or Y is NULL");
    if (!aligned16(X) || !aligned16(Y)) return fail(TSP_ERR_INVALID_ARG, "X and Y must be 16-byte aligned");
    const int64_t es = h->dtype == TSP_DTYPE_BF16 ? 2 : 4;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(X), x1 = x0 + (uintptr_t)(T * h->d * es);
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(Y), y1 = y0 + (uintptr_t)(T * h->d * 4);
    if (x0 < y1 && y0 < x1) return fail(TSP_ERR_INVALID_ARG, "Y overlaps X");
    return TSP_OK;
}

// The forward's launches with the workspace at `work` (hidden activations at
// 0, split partials at pl.part_off). timing = false launches nothing but the
// kernels (no events are created or recorded).
// save: the gate/up accumulators go there too (tile shape 0 only).
tsp_status_t run_forward(tsp_mlp* h, int64_t T, const void* X, float* Y, hipStream_t st, const FwdPlan& pl,
                         void* work, bool timing, float* save = nullptr) {
    const bool swiglu = h->act == TSP_ACT_SWIGLU;
    const bool saved = h->timing;
    h->timing = h->timing && timing;
    struct Restore { tsp_mlp* h; bool v; ~Restore() { h->timing = v; } } restore{h, saved};
    tsp_status_t s;
    if (h->dtype == TSP_DTYPE_BF16) {
        tsp::Bf16Args a;
        a.packed = static_cast<const uint16_t*>(h->packed);
        a.x = static_cast<const uint16_t*>(X);
        a.h = static_cast<uint16_t*>(work);
        a.y = Y;
        a.part = reinterpret_cast<float*>(static_cast<char*>(work) + pl.part_off);
        a.shard_elems = h->shard_elems;
        a.down_off = h->down_off;
        a.T = (int)T; a.d = (int)h->d; a.f = (int)h->f; a.F = (int)h->F; a.P = h->P;
        a.swiglu = swiglu ? 1 : 0;
        a.nbt = pl.nbt;
        a.save = save;
        if (pl.skinny) {
            s = timed_launch(h, "skinny_gateup", st, [&] { return tsp::launch_gateup_skinny(a, st); });
            if (s != TSP_OK) return s;
            return timed_launch(h, "skinny_down", st, [&] { return tsp::launch_down_skinny(a, st); });
        }
        s = timed_launch(h, save ? "gateup_save" : "gateup_tiled", st,
                         [&] { return tsp::launch_gateup_tiled(a, pl.cg, st); });
        if (s != TSP_OK) return s;
        s = timed_launch(h, "down_tiled", st, [&] { return tsp::launch_down_tiled(a, pl.cd, pl.split, st); });
        if (s != TSP_OK || pl.split == 1) return s;
        return timed_launch(h, "reduce_partials", st,
                            [&] { return tsp::launch_reduce_partials(a.part, pl.split, T * a.d, Y, st); });
    }
    tsp::F32Args a;
    a.packed = static_cast<const float*>(h->packed);
    a.x = static_cast<const float*>(X);
    a.h = static_cast<float*>(work);
    a.y = Y;
    a.part = reinterpret_cast<float*>(static_cast<char*>(work) + pl.part_off);
    a.shard_elems = h->shard_elems;
    a.T = (int)T; a.d = (int)h->d; a.f = (int)h->f; a.F = (int)h->F; a.P = h->P;
    a.swiglu = swiglu ? 1 : 0;
    a.split = pl.split;
    s = timed_launch(h, "gateup_f32", st, [&] { return tsp::launch_gateup_f32(a, st); });
    if (s != TSP_OK) return s;
    s = timed_launch(h, "down_f32", st, [&] { return tsp::launch_down_f32(a, st); });
    if (s != TSP_OK || pl.split == 1) return s;
    return timed_launch(h, "reduce_partials", st, [&] { return tsp::launch_reduce_f32(a.part, pl.split, T * a.d, Y, st); });
}

}  // namespace

extern "C" {

tsp_status_t tsp_mlp_forward(tsp_mlp_t h, int64_t T, const void* X, float* Y, hipStream_t stream) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (T < 0 || T > h->T_max) return fail(TSP_ERR_INVALID_ARG, "T=%lld out of [0, T_max=%lld]", (long long)T, (long long)h->T_max);
    if (T == 0) return TSP_OK;
    tsp_status_t s = check_forward_args(h, T, X, Y);
    if (s != TSP_OK) return s;
    FwdPlan pl;
    s = plan_forward(h, T, pl);
    if (s != TSP_OK) return s;
    if (pl.h_bytes > h->part_off || pl.total - pl.part_off > h->work_bytes - h->part_off)
        return fail(TSP_ERR_HIP, "internal: the forward's workspace exceeds the handle's");
    pl.part_off = h->part_off;                  // the handle's layout: partials after T_max tokens of H
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(TSP_ERR_HIP, "cannot select the handle's device");
    return run_forward(h, T, X, Y, stream ? stream : h->stream, pl, h->work, true);
}

}  // extern "C"

namespace {

// ---- the allocation-free forward ----------------------------------------
// Its workspace is this file-scope device array. In host code `scratch` is a
// host-side stand-in, not a device address: host code uses the address that
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr int64_t kStaticScratchBytes = TSP_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device dev (current), looked up once.
tsp_status_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(TSP_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e == hipSuccess ? hipErrorInvalidSymbol : e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TSP_OK;
}

}  // namespace

extern "C" {

tsp_status_t tsp_mlp_forward_static(tsp_mlp_t h, int64_t T, const void* X, float* Y, hipStream_t stream) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (T < 0) return fail(TSP_ERR_INVALID_ARG, "T=%lld is negative", (long long)T);
    if (T == 0) return TSP_OK;
    if (T > kMaxDim) return fail(TSP_ERR_INVALID_ARG, "T=%lld out of range", (long long)T);
    FwdPlan pl;
    tsp_status_t s = plan_forward(h, T, pl);
    if (s != TSP_OK) return s;
    if (pl.total > kStaticScratchBytes)
        return fail(TSP_ERR_UNSUPPORTED, "T=%lld needs %lld bytes of workspace; the static scratch holds %lld",
                    (long long)T, (long long)pl.total, (long long)kStaticScratchBytes);
    s = check_forward_args(h, T, X, Y);
    if (s != TSP_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(TSP_ERR_HIP, "cannot select the handle's device");
    void* work = nullptr;
    s = scratch_address(h->device, &work);
    if (s != TSP_OK) return s;
    return run_forward(h, T, X, Y, stream ? stream : h->stream, pl, work, false);
}

namespace {

// Backward workspace, regions in bytes for T_max tokens (each 256-aligned):
// transposed X and dY (d x Tp), dH (T x f fp32), dG and dU (T x f bf16, for
// dX), dG, dU and H transposed (f x Tp, for the weight gradients), Tp = T_max
// rounded up to 64; then the weights (bf16, row-major Wg, Wu d x f and Wd
// f x d) unpacked from the records.
struct BwdLayout {
    int64_t xt, dyt, dh, dg, du, dgt, dut, ht, wg, wu, wd, wgf, wuf, total;
};

BwdLayout bwd_layout(int64_t T_max, int64_t d, int64_t f) {
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    const int64_t Tp = (T_max + 63) / 64 * 64;
    BwdLayout L;
    int64_t o = 0;
    L.xt = o; o += up(d * Tp * 2);
    L.dyt = o; o += up(d * Tp * 2);
    L.dh = o; o += up(T_max * f * 4);
    L.dg = o; o += up(T_max * f * 2);
    L.du = o; o += up(T_max * f * 2);
    L.dgt = o; o += up(f * Tp * 2);
    L.dut = o; o += up(f * Tp * 2);
    L.ht = o; o += up(f * Tp * 2);
    L.wg = o; o += up(d * f * 2);                   // row-major weights unpacked from the records
    L.wu = o; o += up(d * f * 2);
    L.wd = o; o += up(f * d * 2);
    L.wgf = o; o += up(d * f * 2);                  // Wg, Wu again in fragment blocks (rows d, reduction f)
    L.wuf = o; o += up(d * f * 2);
    L.total = o;
    return L;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

// The backward, from recomputed (saved == nullptr) or saved pre-activations.
static tsp_status_t backward_impl(tsp_mlp_t h, int64_t T, const void* X, const void* dY, const void* saved,
                                  int64_t saved_bytes, float* dX, float* dW_gate, float* dW_up, float* dW_down,
                                  hipStream_t stream) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (T < 0 || T > h->T_max) return fail(TSP_ERR_INVALID_ARG, "T=%lld out of [0, T_max=%lld]", (long long)T, (long long)h->T_max);
    if (h->dtype != TSP_DTYPE_BF16) return fail(TSP_ERR_UNSUPPORTED, "the backward is bf16 only");
    if (h->d % 256 || h->F % 256) return fail(TSP_ERR_UNSUPPORTED, "the backward needs d %% 256 == 0 and F %% 256 == 0");
    if (T == 0) return TSP_OK;
    const bool swiglu = h->act == TSP_ACT_SWIGLU;
    if (!X || !dY || !dX || !dW_up || !dW_down) return fail(TSP_ERR_INVALID_ARG, "a required pointer is NULL");
    if (swiglu != (dW_gate != nullptr))
        return fail(TSP_ERR_INVALID_ARG, "dW_gate is required for SwiGLU and must be NULL for GeLU");
    const void* ptrs[] = {X, dY, dX, dW_gate, dW_up, dW_down};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return fail(TSP_ERR_INVALID_ARG, "every pointer must be 16-byte aligned");
    const int64_t d = h->d, f = h->f;
    struct Span { const void* p; int64_t n; };
    const int64_t need_saved = tsp::gateup_saved_bytes(T, h->F, h->P, swiglu ? 1 : 0);
    if (saved) {
        if (!aligned16(saved)) return fail(TSP_ERR_INVALID_ARG, "every pointer must be 16-byte aligned");
        if (saved_bytes < need_saved)
            return fail(TSP_ERR_INVALID_ARG, "saved holds %lld bytes; T=%lld needs %lld", (long long)saved_bytes,
                        (long long)T, (long long)need_saved);
    }
    const Span outs[] = {{dX, T * d * 4}, {dW_gate, d * f * 4}, {dW_up, d * f * 4}, {dW_down, f * d * 4}};
    const Span ins[] = {{X, T * d * 2}, {dY, T * d * 2}, {saved, saved ? need_saved : 0}};
    for (int i = 0; i < 4; ++i) {
        if (!outs[i].p) continue;
        for (int j = i + 1; j < 4; ++j)
            if (outs[j].p && overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(TSP_ERR_INVALID_ARG, "gradient outputs overlap each other");
        for (const Span& in : ins)
            if (in.p && overlaps(outs[i].p, outs[i].n, in.p, in.n))
                return fail(TSP_ERR_INVALID_ARG, "a gradient output overlaps an input");
    }
    hipStream_t st = stream ? stream : h->stream;
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(TSP_ERR_HIP, "cannot select the handle's device");
    const BwdLayout L = bwd_layout(h->T_max, d, f);
    if (!h->bwd) {
        hipError_t e = hipMalloc(&h->bwd, (size_t)L.total);
        if (e != hipSuccess) {
            h->bwd = nullptr;
            (void)hipGetLastError();
            return fail(TSP_ERR_OOM, "backward workspace of %lld bytes: %s", (long long)L.total, hipGetErrorString(e));
        }
        h->bwd_bytes = L.total;
        h->bwd_unpacked = false;
    }
    char* wsp = static_cast<char*>(h->bwd);
    auto bf = [&](int64_t off) { return reinterpret_cast<uint16_t*>(wsp + off); };
    uint16_t *xt = bf(L.xt), *dyt = bf(L.dyt), *dg = bf(L.dg), *du = bf(L.du);
    uint16_t *dgt = bf(L.dgt), *dut = bf(L.dut), *ht = bf(L.ht);
    float* dh = reinterpret_cast<float*>(wsp + L.dh);
    const int Tp = (int)((T + 63) / 64 * 64);
    const int F = (int)h->F, P = h->P;
    const auto* x16 = static_cast<const uint16_t*>(X);
    const auto* dy16 = static_cast<const uint16_t*>(dY);
    const uint16_t* wgf = swiglu ? bf(L.wgf) : nullptr;
    const uint16_t* wuf = bf(L.wuf);
    const uint16_t* wd16 = bf(L.wd);
    if (!h->bwd_unpacked) {
        // the handle's weights in the layouts the dY and dG / dU products
        // read, once per handle (the records never change): row-major Wd (dH),
        // and Wg, Wu in fragment blocks (dX) by way of row-major copies
        tsp_status_t su = timed_launch(h, "bwd_unpack", st, [&] {
            hipError_t e = tsp::launch_unpack_bf16(h->packed, bf(L.wg), bf(L.wu), bf(L.wd), h->order_dev,
                                                   h->shard_elems, h->down_off, (int)d, (int)f, (int)h->F, h->P,
                                                   swiglu ? 1 : 0, st);
            if (e == hipSuccess && swiglu) e = tsp::launch_pack_frag_bf16(bf(L.wg), f, (int)d, (int)f, bf(L.wgf), st);
            return e != hipSuccess ? e : tsp::launch_pack_frag_bf16(bf(L.wu), f, (int)d, (int)f, bf(L.wuf), st);
        });
        if (su != TSP_OK) return su;
        h->bwd_unpacked = true;
    }

    // dH[t][c] = sum_n dY[t][n] Wd[c][n], natural hidden columns; the same
    // launch transposes X (row-major X^T) and dY (dY^T in fragment blocks)
    // for the weight gradients, on the CUs dH's last partial round leaves idle
    const tsp::TransposeJob tps[2] = {{x16, xt, (int)T, (int)d, (int)d, Tp, 0},
                                      {dy16, dyt, (int)T, (int)d, (int)d, Tp, 1}};
    tsp::NtArgs p{};
    p.a_base[0] = p.a_base[1] = wd16;
    p.b_base[0] = p.b_base[1] = dy16;
    p.lda = (int)d; p.ldb = (int)d; p.M = (int)f; p.N = (int)T;
    p.spp = (int)(d / 32); p.nseg = 1; p.kinds = 1;
    p.out = dh; p.ldc = f;
    tsp_status_t s = timed_launch(h, "bwd_dh", st, [&] { return tsp::launch_nt(&p, 1, st, tps, 2); });
    if (s != TSP_OK) return s;
    // recompute G, U (H) and form dG, dU, H in ring-ordered hidden columns
    tsp::Bf16Args a{};
    a.packed = static_cast<const uint16_t*>(h->packed);
    a.x = x16;
    a.shard_elems = h->shard_elems;
    a.down_off = h->down_off;
    a.T = (int)T; a.d = (int)d; a.f = (int)f; a.F = F; a.P = P;
    a.swiglu = swiglu ? 1 : 0;
    tsp::BwdArgs b{dh, dg, du, dgt, dut, ht, Tp, h->order_dev, static_cast<const float*>(saved)};
    s = timed_launch(h, saved ? "bwd_saved" : "bwd_gateup", st, [&] { return tsp::launch_gateup_bwd(a, b, st); });
    if (s != TSP_OK) return s;
    // dX[t][i] = sum over ring steps k of dG_k[t] . Wg[i][order[k] F ..] + dU_k[t] . Wu[i][..]
    tsp::NtArgs q{};
    q.a_base[0] = swiglu ? wgf : wuf;
    q.a_base[1] = wuf;
    q.a_frag = 1;
    q.b_base[0] = swiglu ? dg : du;
    q.b_base[1] = du;
    q.a_seg = F; q.b_seg = F; q.order = h->order_dev;
    q.lda = (int)f; q.ldb = (int)f; q.M = (int)d; q.N = (int)T;
    q.spp = F / 32; q.kinds = swiglu ? 2 : 1; q.nseg = P * q.kinds;
    q.out = dX; q.ldc = d;
    // weight gradients: reductions over the (zero-padded) token dimension
    auto dw = [&](const uint16_t* at, const uint16_t* bt, int M, int N, float* out, int64_t ldc, int remap) {
        tsp::NtArgs r{};
        r.a_base[0] = r.a_base[1] = at;
        r.b_base[0] = r.b_base[1] = bt;
        r.lda = Tp; r.ldb = Tp; r.M = M; r.N = N;
        r.spp = Tp / 32; r.nseg = 1; r.kinds = 1;
        r.out = out; r.ldc = ldc; r.remap = remap; r.F = F; r.remap_order = h->order_dev;
        r.a_frag = 1;                                   // dG^T, dU^T, dY^T in fragment blocks
        return r;
    };
    // one launch: the weight gradients' tiles first, then dX's (each dX tile
    // reduces over 2f, a weight-gradient tile over T), so that dX tiles start
    // on the CUs the weight gradients' last partial round leaves idle
    tsp::NtArgs ws[tsp::kMaxNt];
    int nw = 0;
    if (swiglu) ws[nw++] = dw(dgt, xt, (int)f, (int)d, dW_gate, f, 1);   // dW_gate[i][c]
    ws[nw++] = dw(dut, xt, (int)f, (int)d, dW_up, f, 1);
    ws[nw++] = dw(dyt, ht, (int)d, (int)f, dW_down, d, 2);               // dW_down[c][n]
    ws[nw++] = q;
    return timed_launch(h, "bwd_dw_dx", st, [&] { return tsp::launch_nt(ws, nw, st); });
}

tsp_status_t tsp_mlp_backward(tsp_mlp_t h, int64_t T, const void* X, const void* dY, float* dX, float* dW_gate,
                              float* dW_up, float* dW_down, hipStream_t stream) {
    return backward_impl(h, T, X, dY, nullptr, 0, dX, dW_gate, dW_up, dW_down, stream);
}

tsp_status_t tsp_mlp_saved_bytes(tsp_mlp_t h, int64_t T, int64_t* bytes) {
    if (!h || !bytes) return fail(TSP_ERR_INVALID_ARG, "handle or bytes is NULL");
    if (T < 0 || T > h->T_max) return fail(TSP_ERR_INVALID_ARG, "T=%lld out of [0, T_max=%lld]", (long long)T, (long long)h->T_max);
    *bytes = tsp::gateup_saved_bytes(T, h->F, h->P, h->act == TSP_ACT_SWIGLU ? 1 : 0);
    return TSP_OK;
}

tsp_status_t tsp_mlp_forward_train(tsp_mlp_t h, int64_t T, const void* X, float* Y, void* saved, int64_t saved_bytes,
                                   hipStream_t stream) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (T < 0 || T > h->T_max) return fail(TSP_ERR_INVALID_ARG, "T=%lld out of [0, T_max=%lld]", (long long)T, (long long)h->T_max);
    if (h->dtype != TSP_DTYPE_BF16) return fail(TSP_ERR_UNSUPPORTED, "saved activations are bf16 only");
    if (h->d % 256 || h->F % 256) return fail(TSP_ERR_UNSUPPORTED, "saved activations need d %% 256 == 0 and F %% 256 == 0");
    if (T == 0) return TSP_OK;
    tsp_status_t s = check_forward_args(h, T, X, Y);
    if (s != TSP_OK) return s;
    if (!saved) return fail(TSP_ERR_INVALID_ARG, "saved is NULL");
    if (!aligned16(saved)) return fail(TSP_ERR_INVALID_ARG, "saved must be 16-byte aligned");
    const int64_t need = tsp::gateup_saved_bytes(T, h->F, h->P, h->act == TSP_ACT_SWIGLU ? 1 : 0);
    if (saved_bytes < need)
        return fail(TSP_ERR_INVALID_ARG, "saved holds %lld bytes; T=%lld needs %lld", (long long)saved_bytes,
                    (long long)T, (long long)need);
    if (overlaps(saved, need, X, T * h->d * 2) || overlaps(saved, need, Y, T * h->d * 4))
        return fail(TSP_ERR_INVALID_ARG, "saved overlaps X or Y");
    FwdPlan pl;
    s = plan_forward(h, T, pl, true);
    if (s != TSP_OK) return s;
    if (pl.h_bytes > h->part_off || pl.total - pl.part_off > h->work_bytes - h->part_off)
        return fail(TSP_ERR_HIP, "internal: the forward's workspace exceeds the handle's");
    pl.part_off = h->part_off;
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(TSP_ERR_HIP, "cannot select the handle's device");
    return run_forward(h, T, X, Y, stream ? stream : h->stream, pl, h->work, true, static_cast<float*>(saved));
}

tsp_status_t tsp_mlp_backward_saved(tsp_mlp_t h, int64_t T, const void* X, const void* dY, const void* saved,
                                    int64_t saved_bytes, float* dX, float* dW_gate, float* dW_up, float* dW_down,
                                    hipStream_t stream) {
    if (h && T > 0 && !saved) return fail(TSP_ERR_INVALID_ARG, "saved is NULL");
    return backward_impl(h, T, X, dY, saved, saved_bytes, dX, dW_gate, dW_up, dW_down, stream);
}

tsp_status_t tsp_mlp_destroy(tsp_mlp_t h) {
    if (!h) return TSP_OK;
    tsp_status_t s = TSP_OK;
    {
        DeviceGuard guard(h->device);
        hipError_t e = hipStreamSynchronize(h->stream);
        if (e != hipSuccess) s = hip_fail(e, "hipStreamSynchronize in destroy");
        for (size_t i = 0; i < h->used; ++i) (void)hipEventSynchronize(h->pool[i].stop);
        release(h);
    }
    return s;
}

tsp_status_t tsp_mlp_set_path(tsp_mlp_t h, int32_t path) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (path != TSP_PATH_AUTO && path != TSP_PATH_TILED && path != TSP_PATH_SKINNY)
        return fail(TSP_ERR_INVALID_ARG, "unknown path %d", path);
    h->path = path;
    return TSP_OK;
}

tsp_status_t tsp_mlp_set_tiles(tsp_mlp_t h, int32_t gateup_tile, int32_t down_tile) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (h->dtype != TSP_DTYPE_BF16) return fail(TSP_ERR_UNSUPPORTED, "tile shapes apply to the bf16 path");
    const bool swiglu = h->act == TSP_ACT_SWIGLU;
    if (gateup_tile >= 0 && !tsp::gateup_cfg_fits(gateup_tile, (int)h->d, (int)h->F, swiglu))
        return fail(TSP_ERR_UNSUPPORTED, "gate/up tile shape %d does not divide the shard", gateup_tile);
    if (down_tile >= 0 && !tsp::down_cfg_fits(down_tile, (int)h->d, (int)h->F))
        return fail(TSP_ERR_UNSUPPORTED, "down tile shape %d does not divide d", down_tile);
    if (gateup_tile < -1 || down_tile < -1) return fail(TSP_ERR_INVALID_ARG, "tile shape < -1");
    h->cfg_gateup = gateup_tile;
    h->cfg_down = down_tile;
    return TSP_OK;
}

tsp_status_t tsp_mlp_sizes(tsp_mlp_t h, int64_t* packed_bytes, int64_t* workspace_bytes) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (packed_bytes) *packed_bytes = h->packed_bytes;
    if (workspace_bytes) *workspace_bytes = h->work_bytes;
    return TSP_OK;
}

tsp_status_t tsp_mlp_set_timing(tsp_mlp_t h, int32_t enable) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    h->timing = enable != 0;
    return TSP_OK;
}

namespace {
tsp_status_t read_timing(tsp_mlp* h, int32_t max_kernels, char (*names)[64], double* total_ms, int64_t* launches,
                         int32_t* n_kernels);
}  // namespace

tsp_status_t tsp_mlp_read_timing(tsp_mlp_t h, int32_t max_kernels, char (*names)[64], double* total_ms,
                                 int64_t* launches, int32_t* n_kernels) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    return read_timing(h, max_kernels, names, total_ms, launches, n_kernels);
}

}  // extern "C"

namespace {
tsp_status_t read_timing(tsp_mlp* h, int32_t max_kernels, char (*names)[64], double* total_ms, int64_t* launches,
                         int32_t* n_kernels) {
    if (max_kernels < 0 || (max_kernels > 0 && (!names || !total_ms || !launches)) || !n_kernels)
        return fail(TSP_ERR_INVALID_ARG, "bad output arrays");
    DeviceGuard guard(h->device);
    tsp_status_t s = drain_timing(h);
    if (s != TSP_OK) return s;
    int32_t n = 0;
    for (KernelTotal& kt : h->totals) {
        if (kt.launches == 0) continue;
        if (n < max_kernels) {
            snprintf(names[n], 64, "%s", kt.name.c_str());
            total_ms[n] = kt.ms;
            launches[n] = kt.launches;
        }
        ++n;
        kt.ms = 0.0;
        kt.launches = 0;
    }
    *n_kernels = n < max_kernels ? n : max_kernels;
    return TSP_OK;
}
}  // namespace

// ---- attention block -------------------------------------------------------

// The attention handle reuses the MLP handle's device, stream, order, event
// timing and buffers: `packed` holds the Q/K/V records, `work` the query and
// attention-output buffers and the split partials of the output projection.
struct tsp_attn : tsp_mlp {
    int32_t H = 0, Hkv = 0, causal = 1;
    int64_t Hs = 0, Hks = 0, Fq = 0, Fqkv = 0, S_pad = 0;
    void* packed_o = nullptr;                  // output-projection records (rows of Wo)
    int64_t packed_o_bytes = 0, rec_qkv = 0, rec_o = 0;
    void* ctx = nullptr;                       // K context (S_pad x Hkv 128), then V^T (Hkv 128 x S_pad)
    int64_t ctx_bytes = 0, o_off = 0;
};

namespace {

void release_attn(tsp_attn* h) {
    if (!h) return;
    free_buffers(h);
    if (h->packed_o) (void)hipFree(h->packed_o);
    if (h->ctx) (void)hipFree(h->ctx);
    delete h;
}

uint16_t* attn_q(tsp_attn* h) { return static_cast<uint16_t*>(h->work); }
uint16_t* attn_o(tsp_attn* h) { return reinterpret_cast<uint16_t*>(static_cast<char*>(h->work) + h->o_off); }
uint16_t* attn_k(tsp_attn* h) { return static_cast<uint16_t*>(h->ctx); }
uint16_t* attn_vt(tsp_attn* h) { return static_cast<uint16_t*>(h->ctx) + h->S_pad * h->Hkv * tsp::ATT_DH; }

tsp_status_t attn_check_call(tsp_attn* h, int64_t T, int32_t rank, const void* X) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (T < 1 || T > h->T_max) return fail(TSP_ERR_INVALID_ARG, "T=%lld out of [1, T_max=%lld]", (long long)T, (long long)h->T_max);
    if (T % 32) return fail(TSP_ERR_UNSUPPORTED, "T=%lld is not a multiple of 32", (long long)T);
    if (rank < 0 || rank >= h->P) return fail(TSP_ERR_INVALID_ARG, "rank=%d out of [0, P=%d)", rank, h->P);
    if (!X) return fail(TSP_ERR_INVALID_ARG, "X is NULL");
    if (!aligned16(X)) return fail(TSP_ERR_INVALID_ARG, "X must be 16-byte aligned");
    return TSP_OK;
}

tsp_status_t attn_project(tsp_attn* h, int64_t T, int32_t rank, const void* X, hipStream_t st) {
    tsp::ProjArgs p;
    p.packed = static_cast<const uint16_t*>(h->packed);
    p.x = static_cast<const uint16_t*>(X);
    p.q = attn_q(h);
    p.kc = attn_k(h);
    p.vt = attn_vt(h);
    p.order = h->order_dev;
    p.rec_elems = h->rec_qkv;
    p.ldq = h->H * tsp::ATT_DH;
    p.ldk = h->Hkv * tsp::ATT_DH;
    p.ldv = h->S_pad;
    p.row0 = (int64_t)rank * T;
    p.T = (int)T; p.d = (int)h->d; p.P = h->P; p.Hs = (int)h->Hs; p.Hks = (int)h->Hks;
    p.q_scale = (float)(1.4426950408889634 / sqrt((double)tsp::ATT_DH));
    return timed_launch(h, "attn_qkv", st, [&] { return tsp::launch_qkv(p, st); });
}

}  // namespace

extern "C" {

tsp_status_t tsp_attn_create(tsp_attn_t* out, int64_t T_max, int64_t d, int32_t H, int32_t Hkv, int32_t dh,
                             int32_t P, int32_t causal, const int32_t* order, const void* w_q, const void* w_k,
                             const void* w_v, const void* w_o, hipStream_t stream) {
    if (!out) return fail(TSP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (T_max < 1 || T_max > kMaxDim) return fail(TSP_ERR_INVALID_ARG, "T_max=%lld out of [1, 2^30]", (long long)T_max);
    if (d < 1 || d > kMaxDim) return fail(TSP_ERR_INVALID_ARG, "d=%lld out of [1, 2^30]", (long long)d);
    if (H < 1 || Hkv < 1 || dh < 1 || P < 1) return fail(TSP_ERR_INVALID_ARG, "H, Hkv, dh and P must be positive");
    if (H % Hkv) return fail(TSP_ERR_INVALID_ARG, "Hkv=%d does not divide H=%d", Hkv, H);
    if (Hkv % P) return fail(TSP_ERR_INVALID_ARG, "P=%d does not divide Hkv=%d", P, Hkv);
    if (order) {
        std::vector<char> seen((size_t)P, 0);
        for (int32_t k = 0; k < P; ++k) {
            const int32_t s = order[k];
            if (s < 0 || s >= P || seen[(size_t)s]) return fail(TSP_ERR_INVALID_ARG, "order is not a permutation of 0..P-1 (entry %d = %d)", k, s);
            seen[(size_t)s] = 1;
        }
    }
    if (!w_q || !w_k || !w_v || !w_o) return fail(TSP_ERR_INVALID_ARG, "weight pointer is NULL");
    if (!aligned16(w_q) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(w_o))
        return fail(TSP_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");
    const int32_t G = H / Hkv;
    if (dh != tsp::ATT_DH) return fail(TSP_ERR_UNSUPPORTED, "dh=%d: the kernels take dh = 128", dh);
    if (!(G == 1 || G == 2 || G % 4 == 0)) return fail(TSP_ERR_UNSUPPORTED, "H/Hkv=%d is not 1, 2 or a multiple of 4", G);
    if ((H / P) % 2) return fail(TSP_ERR_UNSUPPORTED, "H/P=%d is odd", H / P);
    if (d % 256) return fail(TSP_ERR_UNSUPPORTED, "d=%lld is not a multiple of 256", (long long)d);
    // the context's 32-bit buffer offsets span 128 rows of V^T (one head)
    if (P * T_max > (int64_t(1) << 22) || T_max * (int64_t)H * dh > (int64_t(1) << 40) / 2)
        return fail(TSP_ERR_UNSUPPORTED, "T_max too large for this head count");

    tsp_attn* h = new (std::nothrow) tsp_attn;
    if (!h) return fail(TSP_ERR_OOM, "host allocation failed");
    h->T_max = T_max; h->d = d; h->P = P; h->H = H; h->Hkv = Hkv; h->causal = causal ? 1 : 0;
    h->dtype = TSP_DTYPE_BF16; h->stream = stream;
    h->Hs = H / P; h->Hks = Hkv / P;
    h->Fq = h->Hs * dh;
    h->Fqkv = (h->Hs + 2 * h->Hks) * dh;
    h->f = (int64_t)H * dh; h->F = h->Fq;
    h->S_pad = (P * T_max + 63) / 64 * 64;           // positions; each 32-group is stored permuted (attn.hip)
    h->order.resize((size_t)P);
    for (int32_t k = 0; k < P; ++k) h->order[(size_t)k] = order ? order[k] : k;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) { release_attn(h); return hip_fail(e, "hipGetDevice"); }

    h->rec_qkv = d * h->Fqkv;
    h->rec_o = h->Fq * d;
    h->packed_bytes = h->rec_qkv * P * 2;
    h->packed_o_bytes = h->rec_o * P * 2;
    const int64_t qo = (T_max * H * dh * 2 + 255) / 256 * 256;
    h->o_off = qo;
    h->part_off = 2 * qo;
    h->work_bytes = 2 * qo + tsp::down_split_bytes(T_max, (int)d, P);
    h->ctx_bytes = 2 * h->S_pad * Hkv * dh * 2;
    if ((e = hipMalloc(&h->order_dev, sizeof(int32_t) * (size_t)P)) != hipSuccess ||
        (e = hipMalloc(&h->packed, (size_t)h->packed_bytes)) != hipSuccess ||
        (e = hipMalloc(&h->packed_o, (size_t)h->packed_o_bytes)) != hipSuccess ||
        (e = hipMalloc(&h->work, (size_t)h->work_bytes)) != hipSuccess ||
        (e = hipMalloc(&h->ctx, (size_t)h->ctx_bytes)) != hipSuccess) {
        const bool oom = e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation;
        release_attn(h);
        (void)hipGetLastError();
        return oom ? fail(TSP_ERR_OOM, "device allocation of packed weights / workspace / context failed")
                   : hip_fail(e, "hipMalloc");
    }
    e = hipMemcpyAsync(h->order_dev, h->order.data(), sizeof(int32_t) * (size_t)P, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->ctx, 0, (size_t)h->ctx_bytes, stream);
    if (e != hipSuccess) { release_attn(h); return hip_fail(e, "context set-up"); }
    e = tsp::launch_pack_qkv_bf16(w_q, w_k, w_v, h->packed, h->order_dev, h->rec_qkv, (int)d, H, Hkv, dh, P, stream);
    if (e == hipSuccess)
        e = tsp::launch_pack_rows_bf16(w_o, h->packed_o, h->order_dev, h->rec_o, (int)d, (int)h->Fq, P, stream);
    if (e != hipSuccess) { release_attn(h); return hip_fail(e, "pack launch"); }
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) { release_attn(h); return hip_fail(e, "hipStreamSynchronize after packing"); }
    *out = h;
    return TSP_OK;
}

tsp_status_t tsp_attn_project_kv(tsp_attn_t h, int64_t T, int32_t rank, const void* X, hipStream_t stream) {
    tsp_status_t s = attn_check_call(h, T, rank, X);
    if (s != TSP_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(TSP_ERR_HIP, "cannot select the handle's device");
    return attn_project(h, T, rank, X, stream ? stream : h->stream);
}

tsp_status_t tsp_attn_forward(tsp_attn_t h, int64_t T, int32_t rank, const void* X, float* Y, hipStream_t stream) {
    tsp_status_t s = attn_check_call(h, T, rank, X);
    if (s != TSP_OK) return s;
    if (!Y) return fail(TSP_ERR_INVALID_ARG, "Y is NULL");
    if (!aligned16(Y)) return fail(TSP_ERR_INVALID_ARG, "Y must be 16-byte aligned");
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(X), x1 = x0 + (uintptr_t)(T * h->d * 2);
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(Y), y1 = y0 + (uintptr_t)(T * h->d * 4);
    if (x0 < y1 && y0 < x1) return fail(TSP_ERR_INVALID_ARG, "Y overlaps X");
    hipStream_t st = stream ? stream : h->stream;
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(TSP_ERR_HIP, "cannot select the handle's device");

    s = attn_project(h, T, rank, X, st);
    if (s != TSP_OK) return s;

    tsp::AttnArgs a;
    a.q = attn_q(h);
    a.kc = attn_k(h);
    a.vt = attn_vt(h);
    a.o = attn_o(h);
    a.order = h->order_dev;
    a.ldq = h->H * tsp::ATT_DH;
    a.ldk = h->Hkv * tsp::ATT_DH;
    a.ldv = h->S_pad;
    a.T = (int)T; a.S = (int)(h->P * T); a.row0 = (int)(rank * T);
    a.P = h->P; a.Hs = (int)h->Hs; a.Hks = (int)h->Hks; a.causal = h->causal;
    const int G = (int)(h->Hs / h->Hks);
    a.hw = G < 4 ? G : 4;
    a.qs = 4 / a.hw;
    a.n_hq = G / a.hw;
    a.n_qt = (int)((T + 64 * a.qs - 1) / (64 * a.qs));
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)tsp::ATT_DH));
    s = timed_launch(h, "attn_core", st, [&] { return tsp::launch_attn(a, st); });
    if (s != TSP_OK) return s;

    tsp::Bf16Args o;
    o.packed = static_cast<const uint16_t*>(h->packed_o);
    o.x = nullptr;
    o.h = attn_o(h);
    o.y = Y;
    o.part = reinterpret_cast<float*>(static_cast<char*>(h->work) + h->part_off);
    o.shard_elems = h->rec_o;
    o.down_off = 0;
    o.T = (int)T; o.d = (int)h->d; o.f = (int)h->f; o.F = (int)h->Fq; o.P = h->P;
    o.swiglu = 0;
    const int cd = tsp::choose_down_cfg(o.T, o.d, o.F, o.P);
    if (cd < 0) return fail(TSP_ERR_UNSUPPORTED, "no tile shape fits the output projection");
    const int split = tsp::choose_down_split(o.T, o.d, o.P, cd);
    if (split > 1 && (int64_t)split * T * o.d * 4 > h->work_bytes - h->part_off)
        return fail(TSP_ERR_HIP, "internal: split partials exceed the workspace");
    s = timed_launch(h, "attn_out", st, [&] { return tsp::launch_down_tiled(o, cd, split, st); });
    if (s != TSP_OK || split == 1) return s;
    return timed_launch(h, "reduce_partials", st, [&] { return tsp::launch_reduce_partials(o.part, split, T * o.d, Y, st); });
}

tsp_status_t tsp_attn_destroy(tsp_attn_t h) {
    if (!h) return TSP_OK;
    tsp_status_t s = TSP_OK;
    {
        DeviceGuard guard(h->device);
        hipError_t e = hipStreamSynchronize(h->stream);
        if (e != hipSuccess) s = hip_fail(e, "hipStreamSynchronize in destroy");
        for (size_t i = 0; i < h->used; ++i) (void)hipEventSynchronize(h->pool[i].stop);
        release_attn(h);
    }
    return s;
}

tsp_status_t tsp_attn_set_timing(tsp_attn_t h, int32_t enable) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    h->timing = enable != 0;
    return TSP_OK;
}

tsp_status_t tsp_attn_read_timing(tsp_attn_t h, int32_t max_kernels, char (*names)[64], double* total_ms,
                                  int64_t* launches, int32_t* n_kernels) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    return read_timing(h, max_kernels, names, total_ms, launches, n_kernels);
}

tsp_status_t tsp_attn_sizes(tsp_attn_t h, int64_t* packed_bytes, int64_t* workspace_bytes, int64_t* context_bytes) {
    if (!h) return fail(TSP_ERR_INVALID_ARG, "handle is NULL");
    if (packed_bytes) *packed_bytes = h->packed_bytes + h->packed_o_bytes;
    if (workspace_bytes) *workspace_bytes = h->work_bytes;
    if (context_bytes) *context_bytes = h->ctx_bytes;
    return TSP_OK;
}


// ---- ceiling probes -------------------------------------------------------

extern "C++" {
namespace {

// Times `reps` launches of `launch` on `st` with HIP events after one
// untimed launch; returns milliseconds through *ms.
template <class Fn>
tsp_status_t time_probe(hipStream_t st, int reps, Fn&& launch, double* ms) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipEventCreateWithFlags(&e0, hipEventDisableSystemFence);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&e1, hipEventDisableSystemFence);
    if (err == hipSuccess) err = launch();
    if (err == hipSuccess) err = hipEventRecord(e0, st);
    for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch();
    if (err == hipSuccess) err = hipEventRecord(e1, st);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float t = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&t, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (err != hipSuccess) return hip_fail(err, "probe");
    *ms = t;
    return TSP_OK;
}

}  // namespace
}  // extern "C++"

tsp_status_t tsp_probe_hbm_read(int64_t bytes, int32_t reps, hipStream_t stream, double* gb_per_s) {
    if (!gb_per_s) return fail(TSP_ERR_INVALID_ARG, "gb_per_s is NULL");
    if (bytes < (64LL << 20) || bytes > (16LL << 30) || bytes % (64 << 10))
        return fail(TSP_ERR_INVALID_ARG, "bytes=%lld: need 64 MiB .. 16 GiB, a multiple of 64 KiB", (long long)bytes);
    if (reps < 1 || reps > 1000) return fail(TSP_ERR_INVALID_ARG, "reps=%d out of [1, 1000]", reps);
    void* buf = nullptr;
    void* sink = nullptr;
    if (hipMalloc(&buf, (size_t)bytes) != hipSuccess || hipMalloc(&sink, 64) != hipSuccess) {
        (void)hipGetLastError();
        if (buf) (void)hipFree(buf);
        return fail(TSP_ERR_OOM, "probe buffer of %lld bytes", (long long)bytes);
    }
    tsp_status_t s = TSP_OK;
    hipError_t err = hipMemsetAsync(buf, 0, (size_t)bytes, stream);
    double ms = 0.0;
    if (err != hipSuccess) s = hip_fail(err, "hipMemsetAsync");
    else s = time_probe(stream, reps, [&] { return tsp::launch_probe_hbm_read(buf, bytes, sink, stream); }, &ms);
    (void)hipStreamSynchronize(stream);
    (void)hipFree(buf);
    (void)hipFree(sink);
    if (s != TSP_OK) return s;
    *gb_per_s = (double)bytes * reps / (ms * 1e-3) / 1e9;
    return TSP_OK;
}

tsp_status_t tsp_probe_mfma_bf16(int32_t iters, hipStream_t stream, double* tflops) {
    if (!tflops) return fail(TSP_ERR_INVALID_ARG, "tflops is NULL");
    if (iters < 1 || iters > 1000000) return fail(TSP_ERR_INVALID_ARG, "iters=%d out of [1, 1e6]", iters);
    float* sink = nullptr;
    const size_t n = (size_t)tsp::probe_mfma_blocks() * tsp::probe_mfma_threads();
    if (hipMalloc(&sink, n * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(TSP_ERR_OOM, "probe sink");
    }
    double ms = 0.0;
    const int reps = 5;
    tsp_status_t s = time_probe(stream, reps, [&] { return tsp::launch_probe_mfma_bf16(iters, sink, stream); }, &ms);
    (void)hipStreamSynchronize(stream);
    (void)hipFree(sink);
    if (s != TSP_OK) return s;
    *tflops = tsp::probe_mfma_flops(iters) * reps / (ms * 1e-3) / 1e12;
    return TSP_OK;
}

}  // extern "C"
