/*
 * tsp_mlp.h -- C ABI of the MI355X (gfx950) hot path of one rank's gated-MLP
 * block under tensor-and-sequence-parallel (TSP) weight sharding.
 *
 * What the library computes
 * -------------------------
 * "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
 * Training & Inference", Abstract: every rank holds one sequence shard of the
 * tokens and, in the gated MLP, the weight shards travel round a ring while
 * each rank adds every shard's partial output into its own local result.
 * "Tensor Parallelism: Splitting the Math", section "One transformer MLP,
 * split across two GPUs (Megatron-style)": shard s is a block of columns of
 * the first matrix (here the gate and up projections) and the matching block
 * of rows of the second (the down projection); the shards' products are
 * partial sums whose total is the unsplit MLP.
 *
 * On one GPU the ring becomes a loop over shards resident in HBM. For the
 * rank's T tokens X (T x d) and P shards of F = f / P hidden columns each,
 *
 *   Y = sum_{k=0..P-1} H_{order[k]} . Wd[rows of shard order[k], :]
 *   H_s = SiLU(X . Wg[:, cols of s]) * (X . Wu[:, cols of s])     (SwiGLU)
 *   H_s = GeLU_tanh(X . A[:, cols of s])                           (GeLU; A is w_up)
 *
 * with SiLU(g) = g / (1 + e^-g) and GeLU_tanh(u) = 0.5 u (1 + tanh(sqrt(2/pi)
 * (u + 0.044715 u^3))). Shard s owns hidden columns [s*F, (s+1)*F). There are
 * no biases. Products accumulate in fp32; Y is fp32. In the bf16 path the
 * hidden activations are rounded to bf16 (round to nearest even) before the
 * down projection.
 *
 * Layouts: all matrices are dense row-major with no padding. X is T x d in the
 * handle's dtype, Y is T x d fp32, w_gate / w_up are d x f and w_down is f x d
 * (orientation Y = X W, input x output).
 *
 * Errors: every call returns a tsp_status_t and nothing else crosses the ABI
 * (no exceptions, no aborts). Arguments are checked before any HIP call; on a
 * failed check nothing is launched and nothing is allocated.
 * tsp_last_error() returns a message for the calling thread's last failure.
 *
 * Graphs: tsp_mlp_forward, tsp_mlp_forward_static, tsp_mlp_forward_train and,
 * after a first call on the handle (which allocates the backward workspace),
 * tsp_mlp_backward and tsp_mlp_backward_saved only launch kernels on the
 * given stream (with kernel timing off), so they can be captured into a HIP
 * graph on that stream and replayed; a replay reads the buffers' contents at
 * replay time.
 */
#ifndef TSP_MLP_H
#define TSP_MLP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TSP_OK = 0,
    TSP_ERR_INVALID_ARG = 1,   /* null pointer, bad size, order not a permutation, ... */
    TSP_ERR_UNSUPPORTED = 2,   /* a shape the kernels do not tile (see tsp_mlp_validate) */
    TSP_ERR_OOM = 3,           /* device allocation failed; nothing is leaked */
    TSP_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} tsp_status_t;

typedef enum { TSP_ACT_SWIGLU = 0, TSP_ACT_GELU_TANH = 1 } tsp_act_t;

/* storage type of X and the weights; Y is always fp32 */
typedef enum { TSP_DTYPE_F32 = 0, TSP_DTYPE_BF16 = 1 } tsp_dtype_t;

/* forward path selection (tsp_mlp_set_path) */
typedef enum { TSP_PATH_AUTO = 0, TSP_PATH_TILED = 1, TSP_PATH_SKINNY = 2 } tsp_path_t;

typedef struct tsp_mlp* tsp_mlp_t;   /* opaque handle */

/*
 * Pure host check of a create() argument set; makes no HIP call.
 * has_gate: 1 if a gate matrix will be passed. order: host array of P entries
 * or NULL (NULL means 0, 1, ..., P-1).
 * Returns TSP_ERR_INVALID_ARG when: T_max < 1, d < 1, f < 1, P < 1, P does not
 * divide f, act or dtype unknown, order not a permutation of 0..P-1, has_gate
 * differs from (act == SWIGLU).
 * Returns TSP_ERR_UNSUPPORTED (bf16 only) when d or F = f/P is not a multiple
 * of 64. The fp32 path takes any shape.
 */
tsp_status_t tsp_mlp_validate(int64_t T_max, int64_t d, int64_t f, int32_t P,
                              int32_t act, int32_t dtype, const int32_t* order,
                              int32_t has_gate);

/*
 * Create a handle for one rank's block and copy the weights into the
 * library's packed layout. Shards are packed one after another, each as one
 * contiguous record (gate/up columns of the shard, then its down rows), which
 * is the unit a ring step would move between ranks.
 *
 * out      : receives the handle; set to NULL on any failure.
 * T_max    : largest T any forward on this handle will pass (sizes the
 *            workspace: the hidden activations, T_max x f, plus for bf16
 *            up to 64 MiB of fp32 partials for a split down product).
 * d, f, P  : hidden size, FFN width, number of weight shards.
 * act      : tsp_act_t.   dtype: tsp_dtype_t.
 * order    : host array of P int32, the ring order (order[k] = shard used at
 *            step k), a permutation of 0..P-1; NULL = 0..P-1. Copied.
 * w_gate   : device pointer, d x f row-major, dtype; must be NULL for GeLU.
 * w_up     : device pointer, d x f row-major (the matrix A for GeLU).
 * w_down   : device pointer, f x d row-major (the matrix B for GeLU).
 * stream   : HIP stream for the packing kernels; create synchronises it
 *            before returning, so the caller may then free its weights.
 *            It is also the default stream of later forwards.
 * Ownership: the caller keeps its weight buffers; the library owns the packed
 * copy and the workspace until tsp_mlp_destroy. Weight pointers must be
 * 16-byte aligned device memory on the current device.
 */
tsp_status_t tsp_mlp_create(tsp_mlp_t* out, int64_t T_max, int64_t d, int64_t f,
                            int32_t P, int32_t act, int32_t dtype,
                            const int32_t* order, const void* w_gate,
                            const void* w_up, const void* w_down,
                            hipStream_t stream);

/*
 * Y = block(X) for T tokens, visiting the shards in the handle's ring order.
 * X: device, T x d row-major, dtype. Y: device, T x d row-major fp32,
 * overwritten (not accumulated into). Both 16-byte aligned; Y must not
 * overlap X. 0 <= T <= T_max; T == 0 is a no-op.
 * stream: where the kernels run; NULL means the stream given to create.
 * Asynchronous: returns once the kernels are queued. One forward at a time
 * per handle (the hidden-activation workspace is per handle); use one handle
 * per concurrent stream.
 */
tsp_status_t tsp_mlp_forward(tsp_mlp_t h, int64_t T, const void* X, float* Y,
                             hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as tsp_mlp_forward, the same kernels and the same results, with its
 * workspace (hidden activations, down-split partials) in a static device
 * array of TSP_STATIC_SCRATCH_BYTES bytes per GPU instead of the handle's
 * workspace. It allocates nothing and records no timing events. T is bounded
 * by that array, not by T_max: a T whose workspace exceeds it returns
 * TSP_ERR_UNSUPPORTED before any launch (e.g. up to ~2300 tokens at
 * f = 14336 bf16, every T <= 48 of the weight-streaming path). Every call on
 * one GPU shares that GPU's array, which keeps the last call's contents:
 * calls that overlap in time on one GPU (on different streams or host
 * threads) race. The array is set up on the first call on each device and
 * held until the process ends. Arguments and errors otherwise as
 * tsp_mlp_forward.
 */
#define TSP_STATIC_SCRATCH_BYTES (64LL << 20)
tsp_status_t tsp_mlp_forward_static(tsp_mlp_t h, int64_t T, const void* X, float* Y,
                                    hipStream_t stream);

/*
 * Backward of the block for an output gradient dY: the gradients of the
 * forward ("Folding Tensor and Sequence Parallelism ...", Abstract: the method
 * is for training; "Tensor Parallelism: Splitting the Math", the paragraph
 * after the walk-through: the split's synchronisation recurs in the backward
 * pass). For each shard s, in the handle's ring order:
 *   dH_s = dY . Wd_s^T; SwiGLU: dG_s = dH_s * U_s * SiLU'(G_s),
 *   dU_s = dH_s * SiLU(G_s); GeLU: dU_s = dH_s * GeLU'(U_s);
 *   dX += dG_s . Wg_s^T + dU_s . Wu_s^T  (accumulated locally, fp32);
 *   dW_gate[:, s] = X^T . dG_s, dW_up[:, s] = X^T . dU_s,
 *   dW_down[s, :] = H_s^T . dY           (each shard's own blocks),
 * with G_s, U_s, H_s recomputed from X and the handle's packed weights.
 * Every weight the backward reads comes from the handle: the products with dY
 * and with dG / dU read copies that the first backward call unpacks from the
 * packed records (bit-exact) into the backward workspace (Wd row-major, Wg
 * and Wu in the records' fragment-block format transposed), so the gradients
 * always belong to the weights the handle was created with.
 * bf16 handles only (TSP_ERR_UNSUPPORTED for fp32), and d % 256 == 0 and
 * F % 256 == 0 (TSP_ERR_UNSUPPORTED otherwise).
 * X, dY: device, T x d row-major bf16. Outputs, device, fp32, overwritten:
 * dX T x d; dW_gate, dW_up d x f (dW_gate NULL for GeLU, required for
 * SwiGLU); dW_down f x d, the weights' own layouts. All pointers 16-byte
 * aligned; outputs must not overlap each other or the inputs. 1 <= T <= T_max
 * (T == 0 is a no-op). The first call allocates a backward workspace sized
 * for T_max plus the unpacked weights (TSP_ERR_OOM if that fails); it is
 * freed by tsp_mlp_destroy. Asynchronous like forward, on `stream` (NULL: the
 * handle's stream); it shares nothing with a forward's workspace, but one
 * backward at a time per handle.
 */
tsp_status_t tsp_mlp_backward(tsp_mlp_t h, int64_t T, const void* X, const void* dY,
                              float* dX, float* dW_gate, float* dW_up, float* dW_down,
                              hipStream_t stream);

/*
 * The backward from saved pre-activations instead of recomputing them: the
 * same training step ("Folding Tensor and Sequence Parallelism ...",
 * Abstract; "Tensor Parallelism: Splitting the Math", the paragraph after the
 * walk-through) with the gate and up pre-activations G_s, U_s that the
 * forward computes kept in device memory until the backward, trading
 * tsp_mlp_saved_bytes of memory for the backward's recomputation of the
 * gate/up product (a quarter of its matrix work).
 *
 * tsp_mlp_saved_bytes: *bytes = the size of the saved buffer for T tokens
 * (fp32 pre-activations of whole 256-token tiles: P * ceil(T / 256) * n * 256
 * KiB, n = 2F / 256 for SwiGLU, F / 256 for GeLU). TSP_ERR_INVALID_ARG for a
 * NULL argument or T outside [0, T_max].
 *
 * tsp_mlp_forward_train: tsp_mlp_forward (Y bit for bit that of a
 * tsp_mlp_forward on the tiled path with gate/up tile shape 0, the automatic
 * choice at large T, and the same down tile setting) that
 * also writes the pre-activations to `saved`, a caller-owned device buffer of
 * saved_bytes >= tsp_mlp_saved_bytes(T) bytes, 16-byte aligned, overlapping
 * neither X nor Y. Its layout is private to the library. It always runs the
 * gate/up product on the tiled kernel of shape 0 (path and gate/up tile
 * settings do not apply). bf16 handles with d % 256 == 0 and F % 256 == 0
 * (TSP_ERR_UNSUPPORTED otherwise); other errors as tsp_mlp_forward, plus
 * TSP_ERR_INVALID_ARG for a NULL, misaligned, too small or overlapping saved.
 *
 * tsp_mlp_backward_saved: tsp_mlp_backward with the pre-activations read from
 * `saved` (saved_bytes as above), which must hold what tsp_mlp_forward_train
 * wrote for the same handle, T and X (the library cannot check this; other
 * contents give wrong gradients). The gradients are bit for bit those of
 * tsp_mlp_backward. Arguments and errors as tsp_mlp_backward, plus
 * TSP_ERR_INVALID_ARG for a NULL, misaligned or too small saved, or an output
 * overlapping it. saved is only read.
 */
tsp_status_t tsp_mlp_saved_bytes(tsp_mlp_t h, int64_t T, int64_t* bytes);
tsp_status_t tsp_mlp_forward_train(tsp_mlp_t h, int64_t T, const void* X, float* Y, void* saved,
                                   int64_t saved_bytes, hipStream_t stream);
tsp_status_t tsp_mlp_backward_saved(tsp_mlp_t h, int64_t T, const void* X, const void* dY,
                                    const void* saved, int64_t saved_bytes, float* dX, float* dW_gate,
                                    float* dW_up, float* dW_down, hipStream_t stream);

/* Synchronise the handle's stream and free everything it owns. NULL is a no-op. */
tsp_status_t tsp_mlp_destroy(tsp_mlp_t h);

/* Choose the forward path: AUTO (the weight-streaming skinny kernels when
 * T <= 48 and the shape suits them, bf16 only), TILED or SKINNY. SKINNY needs
 * bf16, T <= 48, d % 256 == 0 and P * F % 1024 == 0 at forward time
 * (TSP_ERR_UNSUPPORTED otherwise). */
tsp_status_t tsp_mlp_set_path(tsp_mlp_t h, int32_t path);

/* Tuning and test hook for the bf16 tiled path: fix the tile shape of the
 * gate/up and down kernels (-1 = choose per forward from T and the shape).
 * Shapes (features x tokens): 0 = 256 x 256 with 16x16x32 MFMAs, four waves of
 * 128 x 128 over global-to-LDS loads (the automatic choice at large T),
 * 1 = 256 x 128, 2 = 128 x 128, 3 = 64 x 128 (32x32x16 MFMAs, register-staged
 * loads; for small T and shard widths that are not multiples of 256). With
 * down shape 0 and fewer than 256 output tiles, the ring is split into
 * groups of consecutive shards whose fp32 partials are added in ring order.
 * TSP_ERR_UNSUPPORTED if the shape does not divide the shard's
 * packed width (gate/up) or d (down), or for an fp32 handle. */
tsp_status_t tsp_mlp_set_tiles(tsp_mlp_t h, int32_t gateup_tile, int32_t down_tile);

/* Read back the packed weights' size in bytes and the workspace size in bytes. */
tsp_status_t tsp_mlp_sizes(tsp_mlp_t h, int64_t* packed_bytes, int64_t* workspace_bytes);

/*
 * Kernel timing, for measurement. When enabled, each forward records a pair of
 * HIP events around every kernel it launches, on the stream the kernel runs
 * on. tsp_mlp_read_timing synchronises the handle's event pool, adds up the
 * elapsed time per kernel name since the last read, and resets the sums.
 * names: caller array of max_kernels char buffers of 64 bytes each;
 * total_ms / launches: caller arrays of max_kernels entries; *n_kernels gets
 * the number of distinct kernels filled in.
 */
tsp_status_t tsp_mlp_set_timing(tsp_mlp_t h, int32_t enable);
tsp_status_t tsp_mlp_read_timing(tsp_mlp_t h, int32_t max_kernels, char (*names)[64],
                                 double* total_ms, int64_t* launches, int32_t* n_kernels);

/*
 * Ceiling probes, for reporting the block's kernels against what this GPU
 * sustains beside its datasheet peaks. Not part of the forward path. Each
 * allocates and frees its own device buffers, synchronises `stream` (NULL =
 * the null stream) and times with HIP events recorded on it.
 *
 * tsp_probe_hbm_read: reads a zero-filled device buffer of `bytes` bytes
 * (64 MiB .. 16 GiB, a multiple of 64 KiB) `reps` times (1 .. 1000) with
 * 16-byte nontemporal loads; *gb_per_s = bytes * reps / elapsed / 1e9.
 * tsp_probe_mfma_bf16: every wave issues `iters` (1 .. 1e6) rounds of 16
 * independent v_mfma_f32_16x16x32_bf16 on pseudo-random unit-scale operands,
 * enough waves to fill every SIMD twice over; *tflops = flops / elapsed / 1e12.
 * Errors: TSP_ERR_INVALID_ARG for out-of-range arguments or NULL outputs,
 * TSP_ERR_OOM if the buffer cannot be allocated, TSP_ERR_HIP otherwise.
 */
tsp_status_t tsp_probe_hbm_read(int64_t bytes, int32_t reps, hipStream_t stream, double* gb_per_s);
tsp_status_t tsp_probe_mfma_bf16(int32_t iters, hipStream_t stream, double* tflops);

/* Static text for a status code. */
const char* tsp_status_string(tsp_status_t s);

/* Message of the calling thread's last failed call ("" if none). */
const char* tsp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TSP_MLP_H */
