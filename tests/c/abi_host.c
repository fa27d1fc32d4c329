/* A plain C99 caller of libgsfp8 through include/gs.h: compiled with
 * -std=c99 -Wall -Wextra -pedantic -Werror and linked against the library,
 * it calls the host-only entry points (status strings, workspace sizes, the
 * chunk descriptors of a gradient list) and argument checks that return
 * before any HIP call.  Prints one line per check; exit status 0 when all
 * pass. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gs.h"

static int failures = 0;

static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) ++failures;
}

int main(void) {
    /* status strings start with the status name */
    check(strncmp(gs_status_string(GS_OK), "GS_OK", 5) == 0, "status string GS_OK");
    check(strncmp(gs_status_string(GS_ERR_WORKSPACE), "GS_ERR_WORKSPACE", 16) == 0,
          "status string GS_ERR_WORKSPACE");

    /* workspace sizes */
    check(fp8_quantize_workspace_size(8192, 8192, FP8_PER_TENSOR) == 32768,
          "per-tensor workspace 32 KiB");
    check(fp8_quantize_workspace_size(8192, 8192, FP8_BLOCK_1x128) == 0, "1x128 needs none");
    {
        const int64_t numels[3] = {1, 2048, 2049};
        check(gs_unscale_check_sumsq_workspace_size(3, numels) == 16u * (1 + 1 + 2 + 1024),
              "sum-of-squares workspace = 16 B per chunk + 1024 partials");
    }

    /* chunk descriptors of a two-tensor list at made-up (never dereferenced)
     * 16-byte aligned addresses: 4096 elements (two whole chunks), then 3000
     * (one whole chunk and a ragged one of 952) */
    {
        const void *grads[2] = {(const void *)(uintptr_t)0x100000u, (const void *)(uintptr_t)0x200000u};
        float *outs[2] = {(float *)(uintptr_t)0x300000u, (float *)(uintptr_t)0x400000u};
        const int64_t numels[2] = {4096, 3000};
        uint64_t d[8];
        const int64_t count = gs_unscale_list_descriptors(2, grads, outs, numels, NULL, 0);
        const int64_t got = gs_unscale_list_descriptors(2, grads, outs, numels, d, 4);
        check(count == 4 && got == 4, "four chunks, counted and written");
        check(d[0] == 0x100000u && d[1] == 0x300000u, "chunk 0: whole, aligned");
        check(d[2] == 0x100000u + 4096u && d[3] == 0x300000u + 8192u, "chunk 1: next 2048 elements");
        check(d[4] == 0x200000u && d[5] == 0x400000u, "chunk 2: second tensor");
        check(d[6] == ((uint64_t)952 << 48 | (0x200000u + 4096u)) && d[7] == 0x400000u + 8192u,
              "chunk 3: ragged, 952 elements in bits 48-63");
        check(gs_unscale_list_descriptors(2, grads, outs, numels, d, 3) == GS_ERR_SIZE,
              "capacity too small -> GS_ERR_SIZE");
    }

    /* argument checks (no HIP call is reached) */
    {
        const void *fake = (const void *)(uintptr_t)((uint64_t)1 << 40);
        float *ffake = (float *)(uintptr_t)((uint64_t)1 << 40);
        int32_t *ifake = (int32_t *)(uintptr_t)((uint64_t)1 << 40);
        uint8_t *cfake = (uint8_t *)(uintptr_t)((uint64_t)1 << 40);
        check(fp8_quantize(fake, GS_F16, 128, 128, FP8_E4M3, FP8_BLOCK_1x128, FP8_SCALE_FROM_AMAX,
                           cfake, ffake, NULL, NULL, 0, NULL) == GS_ERR_DTYPE, "FP16 quantize -> GS_ERR_DTYPE");
        check(fp8_quantize(fake, GS_BF16, 128, 100, FP8_E4M3, FP8_BLOCK_1x128, FP8_SCALE_FROM_AMAX,
                           cfake, ffake, NULL, NULL, 0, NULL) == GS_ERR_SHAPE, "1x128 with cols 100 -> GS_ERR_SHAPE");
        check(fp8_quantize(fake, GS_BF16, 64, 64, FP8_E4M3, FP8_PER_TENSOR, FP8_SCALE_FROM_AMAX,
                           cfake, ffake, NULL, NULL, 0, NULL) == GS_ERR_WORKSPACE,
              "per-tensor without workspace -> GS_ERR_WORKSPACE");
        check(gs_update_scale(ffake, ifake, ifake, 2.0f, 0.5f, 0, NULL, NULL) == GS_ERR_ARG,
              "growth interval 0 -> GS_ERR_ARG");
        check(gs_unscale_check(-1, NULL, NULL, NULL, GS_F16, ffake, ifake, NULL) == GS_ERR_SIZE,
              "negative tensor count -> GS_ERR_SIZE");
        check(gs_unscale_check(0, NULL, NULL, NULL, GS_F16, ffake, ifake, NULL) == GS_OK,
              "empty list -> GS_OK, nothing launched");
    }
    printf("%d failure(s)\n", failures);
    return failures != 0;
}
