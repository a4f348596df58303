/*
 * Host-only walk through the C ABI's error paths (no GPU needed: every call
 * here is rejected by argument validation before any HIP call). Built with
 * AddressSanitizer by tests/test_c_abi.py to check the library's host code for
 * memory errors on these paths. Exits 0 when every call returns the expected
 * status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tsp_mlp.h"
#include "tsp_attn.h"

static int failures = 0;

static void expect(const char* what, tsp_status_t got, tsp_status_t want) {
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d; last error: %s\n", what, got, tsp_status_string(got), want,
               tsp_last_error());
        ++failures;
    }
}

int main(void) {
    const int32_t good_order[4] = {2, 3, 0, 1}, dup_order[4] = {0, 1, 1, 2}, neg_order[2] = {0, -1};
    void* fake = (void*)0x1000;
    tsp_mlp_t h = (tsp_mlp_t)0x1;

    expect("valid shape", tsp_mlp_validate(64, 256, 1024, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, good_order, 1), TSP_OK);
    expect("T_max 0", tsp_mlp_validate(0, 256, 1024, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, NULL, 1), TSP_ERR_INVALID_ARG);
    expect("P does not divide f", tsp_mlp_validate(8, 256, 1000, 3, TSP_ACT_SWIGLU, TSP_DTYPE_F32, NULL, 1),
           TSP_ERR_INVALID_ARG);
    expect("duplicate in order", tsp_mlp_validate(8, 256, 1024, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, dup_order, 1),
           TSP_ERR_INVALID_ARG);
    expect("negative in order", tsp_mlp_validate(8, 64, 128, 2, TSP_ACT_SWIGLU, TSP_DTYPE_F32, neg_order, 1),
           TSP_ERR_INVALID_ARG);
    expect("gate with GeLU", tsp_mlp_validate(8, 256, 1024, 4, TSP_ACT_GELU_TANH, TSP_DTYPE_BF16, NULL, 1),
           TSP_ERR_INVALID_ARG);
    expect("no gate with SwiGLU", tsp_mlp_validate(8, 256, 1024, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, NULL, 0),
           TSP_ERR_INVALID_ARG);
    expect("unknown activation", tsp_mlp_validate(8, 256, 1024, 4, 7, TSP_DTYPE_BF16, NULL, 1), TSP_ERR_INVALID_ARG);
    expect("unknown dtype", tsp_mlp_validate(8, 256, 1024, 4, TSP_ACT_SWIGLU, 5, NULL, 1), TSP_ERR_INVALID_ARG);
    expect("bf16 F not a multiple of 64", tsp_mlp_validate(8, 256, 1024, 32, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, NULL, 1),
           TSP_ERR_UNSUPPORTED);
    expect("bf16 d not a multiple of 64", tsp_mlp_validate(8, 200, 1024, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, NULL, 1),
           TSP_ERR_UNSUPPORTED);
    expect("workspace too large", tsp_mlp_validate(1 << 30, 256, 1 << 20, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, NULL, 1),
           TSP_ERR_UNSUPPORTED);

    expect("create: out NULL", tsp_mlp_create(NULL, 8, 64, 128, 2, TSP_ACT_SWIGLU, TSP_DTYPE_F32, NULL, fake, fake,
                                              fake, NULL), TSP_ERR_INVALID_ARG);
    expect("create: bad order", tsp_mlp_create(&h, 8, 256, 1024, 4, TSP_ACT_SWIGLU, TSP_DTYPE_BF16, dup_order, fake,
                                               fake, fake, NULL), TSP_ERR_INVALID_ARG);
    if (h != NULL) { printf("FAIL create did not clear *out\n"); ++failures; }
    expect("create: NULL weight", tsp_mlp_create(&h, 8, 64, 128, 2, TSP_ACT_SWIGLU, TSP_DTYPE_F32, NULL, fake, NULL,
                                                 fake, NULL), TSP_ERR_INVALID_ARG);
    expect("create: misaligned weight", tsp_mlp_create(&h, 8, 64, 128, 2, TSP_ACT_SWIGLU, TSP_DTYPE_F32, NULL, fake,
                                                       (char*)fake + 2, fake, NULL), TSP_ERR_INVALID_ARG);

    expect("forward: NULL handle", tsp_mlp_forward(NULL, 1, fake, (float*)fake, NULL), TSP_ERR_INVALID_ARG);
    expect("destroy: NULL handle", tsp_mlp_destroy(NULL), TSP_OK);
    expect("forward_train: NULL handle", tsp_mlp_forward_train(NULL, 1, fake, (float*)fake, fake, 1 << 20, NULL),
           TSP_ERR_INVALID_ARG);
    expect("backward_saved: NULL handle", tsp_mlp_backward_saved(NULL, 1, fake, fake, fake, 1 << 20, (float*)fake,
                                                                 (float*)fake, (float*)fake, (float*)fake, NULL),
           TSP_ERR_INVALID_ARG);
    int64_t nb = 0;
    expect("saved_bytes: NULL handle", tsp_mlp_saved_bytes(NULL, 1, &nb), TSP_ERR_INVALID_ARG);
    expect("set_path: NULL handle", tsp_mlp_set_path(NULL, 0), TSP_ERR_INVALID_ARG);
    expect("set_tiles: NULL handle", tsp_mlp_set_tiles(NULL, 5, 5), TSP_ERR_INVALID_ARG);
    expect("set_timing: NULL handle", tsp_mlp_set_timing(NULL, 1), TSP_ERR_INVALID_ARG);
    int64_t a = 0, b = 0;
    expect("sizes: NULL handle", tsp_mlp_sizes(NULL, &a, &b), TSP_ERR_INVALID_ARG);
    int32_t n = 0;
    expect("read_timing: NULL handle", tsp_mlp_read_timing(NULL, 0, NULL, NULL, NULL, &n), TSP_ERR_INVALID_ARG);
    double r = 0.0;
    expect("probe_hbm_read: bad size", tsp_probe_hbm_read(1000, 1, NULL, &r), TSP_ERR_INVALID_ARG);
    expect("probe_mfma: bad iters", tsp_probe_mfma_bf16(0, NULL, &r), TSP_ERR_INVALID_ARG);

    /* the attention block's host checks */
    tsp_attn_t ah = (tsp_attn_t)0x1;
    expect("attn create: out NULL", tsp_attn_create(NULL, 64, 4096, 32, 8, 128, 8, 1, NULL, fake, fake, fake, fake,
                                                    NULL), TSP_ERR_INVALID_ARG);
    expect("attn create: Hkv does not divide H", tsp_attn_create(&ah, 64, 4096, 32, 6, 128, 2, 1, NULL, fake, fake,
                                                                  fake, fake, NULL), TSP_ERR_INVALID_ARG);
    if (ah != NULL) { printf("FAIL attn create: *out not cleared\n"); ++failures; }
    expect("attn create: P does not divide Hkv", tsp_attn_create(&ah, 64, 4096, 32, 8, 128, 3, 1, NULL, fake, fake,
                                                                  fake, fake, NULL), TSP_ERR_INVALID_ARG);
    expect("attn create: bad order", tsp_attn_create(&ah, 64, 4096, 32, 8, 128, 4, 1, dup_order, fake, fake, fake,
                                                     fake, NULL), TSP_ERR_INVALID_ARG);
    expect("attn create: NULL weight", tsp_attn_create(&ah, 64, 4096, 32, 8, 128, 8, 1, NULL, fake, NULL, fake, fake,
                                                       NULL), TSP_ERR_INVALID_ARG);
    expect("attn create: dh 64", tsp_attn_create(&ah, 64, 4096, 32, 8, 64, 8, 1, NULL, fake, fake, fake, fake, NULL),
           TSP_ERR_UNSUPPORTED);
    expect("attn create: d 4000", tsp_attn_create(&ah, 64, 4000, 32, 8, 128, 8, 1, NULL, fake, fake, fake, fake,
                                                  NULL), TSP_ERR_UNSUPPORTED);
    expect("attn forward: NULL handle", tsp_attn_forward(NULL, 32, 0, fake, (float*)fake, NULL), TSP_ERR_INVALID_ARG);
    expect("attn project_kv: NULL handle", tsp_attn_project_kv(NULL, 32, 0, fake, NULL), TSP_ERR_INVALID_ARG);
    expect("attn destroy: NULL handle", tsp_attn_destroy(NULL), TSP_OK);
    expect("attn set_timing: NULL handle", tsp_attn_set_timing(NULL, 1), TSP_ERR_INVALID_ARG);
    int64_t c = 0;
    expect("attn sizes: NULL handle", tsp_attn_sizes(NULL, &a, &b, &c), TSP_ERR_INVALID_ARG);
    expect("attn read_timing: NULL handle", tsp_attn_read_timing(NULL, 0, NULL, NULL, NULL, &n), TSP_ERR_INVALID_ARG);

    /* long messages stay bounded and NUL-terminated */
    for (int i = 0; i < 1000; ++i) tsp_mlp_validate(-i, -i, -i, -i, -i, -i, NULL, i & 1);
    if (strlen(tsp_last_error()) == 0 || strlen(tsp_last_error()) > 4096) { printf("FAIL last_error\n"); ++failures; }
    for (int s = -1; s < 8; ++s)
        if (!tsp_status_string((tsp_status_t)s)) { printf("FAIL status string %d\n", s); ++failures; }

    printf("abi_validate: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}
