/*
 * Plain-C use of the tsp_mlp C ABI, with no Python and no PyTorch: device
 * buffers from hipMalloc, one SwiGLU block with identity weights (d = f), so
 * Y = SiLU(X) * X elementwise ("Tensor Parallelism: Splitting the Math",
 * section "Why the column-then-row split": the nonlinearity acts on each
 * hidden column, and identity matrices route hidden column i to output i).
 * Prints the largest error against the host value and exits 0 when every
 * output is within bf16 rounding of the hidden activations (2^-8 relative).
 *
 * Usage: abi_demo [T] (default 40 tokens; d = f = 256, P = 4, ring from shard 1)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tsp_mlp.h"

static uint16_t to_bf16(float x) {          /* round to nearest even; inputs are finite */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

#define HIP_OK(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) { \
    fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); return 2; } } while (0)

int main(int argc, char** argv) {
    const int64_t T = argc > 1 ? atoll(argv[1]) : 40, d = 256, f = 256;
    const int32_t P = 4, order[4] = {1, 2, 3, 0};
    uint16_t* hx = malloc(sizeof(uint16_t) * (size_t)(T * d));
    uint16_t* hw = calloc((size_t)(d * f), sizeof(uint16_t));
    float* hy = malloc(sizeof(float) * (size_t)(T * d));
    if (!hx || !hw || !hy) return 2;
    uint32_t s = 12345u;
    for (int64_t i = 0; i < T * d; ++i) {   /* values in [-4, 4) */
        s = s * 1664525u + 1013904223u;
        hx[i] = to_bf16(((float)(s >> 8) / 16777216.0f) * 8.0f - 4.0f);
    }
    for (int64_t i = 0; i < d; ++i) hw[i * f + i] = to_bf16(1.0f);

    void *dx, *dw, *dy;
    HIP_OK(hipMalloc(&dx, sizeof(uint16_t) * (size_t)(T * d)));
    HIP_OK(hipMalloc(&dw, sizeof(uint16_t) * (size_t)(d * f)));
    HIP_OK(hipMalloc(&dy, sizeof(float) * (size_t)(T * d)));
    HIP_OK(hipMemcpy(dx, hx, sizeof(uint16_t) * (size_t)(T * d), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dw, hw, sizeof(uint16_t) * (size_t)(d * f), hipMemcpyHostToDevice));

    tsp_mlp_t h = NULL;
    tsp_status_t st = tsp_mlp_create(&h, T, d, f, P, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, order, dw, dw, dw, NULL);
    if (st != TSP_OK) { fprintf(stderr, "create: %s: %s\n", tsp_status_string(st), tsp_last_error()); return 2; }
    st = tsp_mlp_forward(h, T, dx, (float*)dy, NULL);
    if (st != TSP_OK) { fprintf(stderr, "forward: %s: %s\n", tsp_status_string(st), tsp_last_error()); return 2; }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hy, dy, sizeof(float) * (size_t)(T * d), hipMemcpyDeviceToHost));
    if (tsp_mlp_destroy(h) != TSP_OK) return 2;

    double worst = 0.0;
    int bad = 0;
    for (int64_t i = 0; i < T * d; ++i) {
        const double x = from_bf16(hx[i]);
        const double want = x / (1.0 + exp(-x)) * x;
        const double err = fabs((double)hy[i] - want);
        const double tol = ldexp(fabs(want), -8) + 1e-6;
        if (err > worst) worst = err;
        if (err > tol) ++bad;
    }
    printf("abi_demo: T=%lld d=%lld outputs=%lld max_abs_err=%.3e out_of_tolerance=%d\n", (long long)T,
           (long long)d, (long long)(T * d), worst, bad);
    hipFree(dx); hipFree(dw); hipFree(dy);
    free(hx); free(hw); free(hy);
    return bad ? 1 : 0;
}
