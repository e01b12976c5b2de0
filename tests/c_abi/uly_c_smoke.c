/*
 * A C program that uses libuly.so through include/uly.h alone (no Python):
 * the Ulysses scatter of a small coordinate-coded tensor and its inverse
 * gather, checked word for word against the CPU oracle (test infrastructure,
 * linked only here), plus the rejection of a head count that does not
 * divide by the world size.  Prints "ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "uly.h"

/* from oracle/uly_oracle.c */
int oracle_scatter(const void *x, void *y, size_t es, int64_t P, int64_t B, int64_t S_l, int64_t H, int64_t D);
int oracle_gather(const void *o, void *z, size_t es, int64_t P, int64_t B, int64_t S, int64_t Hl, int64_t D);

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
            return 1;                                                             \
        }                                                                         \
    } while (0)
#define CHECK_ULY(x)                                                              \
    do {                                                                          \
        uly_status s_ = (x);                                                      \
        if (s_ != ULY_OK) {                                                       \
            fprintf(stderr, "%s: %s %s\n", #x, uly_status_string(s_), uly_last_error()); \
            return 1;                                                             \
        }                                                                         \
    } while (0)

int main(void) {
    enum { P = 4, B = 2, S_l = 37, H = 8, D = 64 };
    const int64_t n = (int64_t)P * B * S_l * H * D;
    const size_t bytes = (size_t)n * 2;
    uint16_t *x = malloc(bytes), *y = malloc(bytes), *z = malloc(bytes), *want = malloc(bytes);
    for (int64_t i = 0; i < n; ++i) x[i] = (uint16_t)(i * 2654435761u >> 7);

    void *x_d = NULL, *y_d = NULL, *z_d = NULL;
    CHECK_HIP(hipMalloc(&x_d, bytes));
    CHECK_HIP(hipMalloc(&y_d, bytes));
    CHECK_HIP(hipMalloc(&z_d, bytes));
    CHECK_HIP(hipMemcpy(x_d, x, bytes, hipMemcpyHostToDevice));

    uly_ctx *ctx = NULL;
    CHECK_ULY(uly_create(&ctx, 0, P, 12));
    const int64_t tshape[4] = {B, (int64_t)P * S_l, H / P, D};
    CHECK_ULY(uly_target_register(ctx, "v", ULY_MODE_SCATTER, ULY_BF16, tshape, y_d, bytes));

    uly_tensor xv;
    memset(&xv, 0, sizeof xv);
    xv.data = x_d;
    xv.dtype = ULY_BF16;
    xv.rank_stride = (int64_t)B * S_l * H * D;
    xv.shape[0] = B; xv.shape[1] = S_l; xv.shape[2] = H; xv.shape[3] = D;
    xv.stride[0] = (int64_t)S_l * H * D; xv.stride[1] = (int64_t)H * D; xv.stride[2] = D; xv.stride[3] = 1;
    const char *tags[3] = {NULL, NULL, "v"};
    CHECK_ULY(ulysses_scatter_qkv(ctx, NULL, NULL, &xv, tags, NULL, 0));
    CHECK_ULY(uly_wait(ctx, 0));

    /* the inverse straight back into an explicit destination */
    uly_tensor yv = xv;
    yv.data = y_d;
    yv.rank_stride = (int64_t)B * P * S_l * (H / P) * D;
    yv.shape[1] = (int64_t)P * S_l; yv.shape[2] = H / P;
    yv.stride[0] = (int64_t)P * S_l * (H / P) * D; yv.stride[1] = (int64_t)(H / P) * D;
    CHECK_ULY(ulysses_gather_out(ctx, &yv, NULL, z_d, 0));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(y, y_d, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(z, z_d, bytes, hipMemcpyDeviceToHost));

    if (oracle_scatter(x, want, 2, P, B, S_l, H, D) != 0 || memcmp(y, want, bytes) != 0) {
        fprintf(stderr, "scatter differs from the oracle\n");
        return 1;
    }
    if (oracle_gather(y, want, 2, P, B, (int64_t)P * S_l, H / P, D) != 0 || memcmp(z, want, bytes) != 0 ||
        memcmp(z, x, bytes) != 0) {
        fprintf(stderr, "gather differs from the oracle or from the input\n");
        return 1;
    }

    /* heads not divisible by the world size: rejected before any launch, context still usable */
    xv.shape[2] = 6;
    void *outs[3] = {NULL, NULL, z_d};
    if (ulysses_scatter_qkv(ctx, NULL, NULL, &xv, tags, outs, 0) != ULY_E_INVAL) {
        fprintf(stderr, "H %% P != 0 was not rejected\n");
        return 1;
    }
    xv.shape[2] = H;
    CHECK_ULY(ulysses_scatter_qkv(ctx, NULL, NULL, &xv, tags, NULL, 0));
    CHECK_ULY(uly_wait(ctx, 0));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_ULY(uly_destroy(ctx));
    CHECK_HIP(hipFree(x_d));
    CHECK_HIP(hipFree(y_d));
    CHECK_HIP(hipFree(z_d));
    free(x); free(y); free(z); free(want);
    printf("ok\n");
    return 0;
}
