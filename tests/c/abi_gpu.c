/* A plain C11 caller of libgsfp8 on the GPU, through include/gs.h only:
 * device buffers from hipMalloc, work on a stream of its own, results copied
 * back and compared bit for bit with the oracle (oracle/oracle.c, linked as
 * oracle/_build/liboracle.so).  Covers the unscale + update, the unscale
 * with the exact sum of squares, the hysteresis update, quantize and
 * dequantize (FP32 and BF16 output) at every granularity in both formats,
 * the MX blocks and three delayed-scaling steps.  Every shape is checked on
 * the host by the library before anything is enqueued.  Prints one line per
 * check and "N failure(s)"; exit status 0 when all pass, 3 on a HIP error. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gs.h"

/* the oracle's functions (oracle/oracle.c) */
void orc_unscale_check(int32_t n, const uint16_t *const *grads, float *const *outs,
                       const int64_t *numels, float S, int32_t *found_inf);
void orc_unscale_check_sumsq(int32_t n, const uint16_t *const *grads, float *const *outs,
                             const int64_t *numels, float S, int32_t *found_inf,
                             uint64_t *sumsq, double *norm_sq);
void orc_update_scale(float *S, int32_t *tracker, int32_t *found_inf, float growth,
                      float backoff, int32_t interval, int64_t *skips);
void orc_update_scale_hysteresis(float *S, int32_t *tracker, int32_t *h, int32_t *found_inf,
                                 float growth, float backoff, int32_t window, int32_t H,
                                 int32_t consecutive, float min_scale, int64_t *skips);
int orc_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int gran,
                 int mode, uint8_t *codes, float *scales, int32_t *nonfinite);
int orc_quantize_delayed(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                         float *scale_state, float *history, int32_t hlen, int32_t *pos,
                         uint8_t *codes, float *scale_used, int32_t *nonfinite);
int orc_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, int fmt, int gran,
                   const float *scales, float *out);
int orc_dequantize_bf16(const uint8_t *codes, int64_t rows, int64_t cols, int fmt, int gran,
                        const float *scales, uint16_t *out);
int orc_quantize_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                    uint8_t *codes, uint8_t *scales_e8m0, int32_t *nonfinite);
int orc_dequantize_mx(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                      const uint8_t *scales_e8m0, float *out);

#define HIPCHECK(call)                                                                   \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            printf("HIP error %d (%s) at %s:%d\n", (int)e_, hipGetErrorString(e_),       \
                   __FILE__, __LINE__);                                                  \
            exit(3);                                                                     \
        }                                                                                \
    } while (0)

static int failures = 0;
static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) ++failures;
}

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint32_t rnd(void) {                       /* xorshift64*, test inputs only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        printf("out of memory\n");
        exit(2);
    }
    return p;
}

static void *to_dev(const void *h, size_t n) {
    void *d = NULL;
    HIPCHECK(hipMalloc(&d, n ? n : 16));
    if (n && h) HIPCHECK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

static void from_dev(void *h, const void *d, size_t n) {
    if (n) HIPCHECK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
}

/* ------------------------------------------------------------ loss scaling */
static void test_unscale(hipStream_t st) {
    enum { N = 5 };
    const int64_t numel[N] = {5000, 2048, 777, 0, 1};
    uint16_t *hg[N];
    float *ho[N], *ref[N];
    const void *dg[N];
    float *dout[N];
    for (int t = 0; t < N; ++t) {
        hg[t] = (uint16_t *)xmalloc((size_t)numel[t] * 2);
        ho[t] = (float *)xmalloc((size_t)numel[t] * 4);
        ref[t] = (float *)xmalloc((size_t)numel[t] * 4);
        for (int64_t i = 0; i < numel[t]; ++i) {
            uint16_t h = (uint16_t)(rnd() & 0xBFFFu);          /* exponent < 16: finite */
            hg[t][i] = h;
        }
        dg[t] = to_dev(hg[t], (size_t)numel[t] * 2);
        dout[t] = (float *)to_dev(NULL, (size_t)numel[t] * 4);
    }
    float S = 65536.0f, hS = 0.0f;
    int32_t tracker = 0, found = 0, hfound = 0, htracker = 0;
    int64_t skips = 0, hskips = 0;
    float *dS = (float *)to_dev(&S, 4);
    int32_t *dtr = (int32_t *)to_dev(&tracker, 4), *dfound = (int32_t *)to_dev(&found, 4);
    int64_t *dskips = (int64_t *)to_dev(&skips, 8);
    /* three steps, an Inf in tensor 1 on the second */
    for (int step = 0; step < 3; ++step) {
        const uint16_t saved = hg[1][100];
        if (step == 1) {
            hg[1][100] = 0x7C00u;
            HIPCHECK(hipMemcpy((uint16_t *)dg[1] + 100, &hg[1][100], 2, hipMemcpyHostToDevice));
        }
        check(gs_unscale_check(N, dg, dout, numel, GS_F16, dS, dfound, st) == GS_OK,
              "gs_unscale_check returns GS_OK");
        HIPCHECK(hipStreamSynchronize(st));
        from_dev(&hfound, dfound, 4);
        int ok = 1;
        orc_unscale_check(N, (const uint16_t *const *)hg, ref, numel, S, &found);
        for (int t = 0; t < N; ++t) {
            from_dev(ho[t], dout[t], (size_t)numel[t] * 4);
            ok &= memcmp(ho[t], ref[t], (size_t)numel[t] * 4) == 0;
        }
        check(ok, "unscale outputs bit-identical to the oracle");
        check(hfound == found, "found_inf matches the oracle");
        check(gs_update_scale(dS, dtr, dfound, 2.0f, 0.5f, 2, dskips, st) == GS_OK,
              "gs_update_scale returns GS_OK");
        orc_update_scale(&S, &tracker, &found, 2.0f, 0.5f, 2, &skips);
        HIPCHECK(hipStreamSynchronize(st));
        from_dev(&hS, dS, 4);
        from_dev(&htracker, dtr, 4);
        from_dev(&hskips, dskips, 8);
        from_dev(&hfound, dfound, 4);
        check(memcmp(&hS, &S, 4) == 0 && htracker == tracker && hskips == skips &&
                  hfound == 0 && found == 0,
              "scaler state matches the oracle");
        if (step == 1) {
            hg[1][100] = saved;
            HIPCHECK(hipMemcpy((uint16_t *)dg[1] + 100, &saved, 2, hipMemcpyHostToDevice));
        }
    }
    check(S == 32768.0f && skips == 1, "closed form: one skip halves S");

    /* the exact sum of squares, added to a running total */
    {
        uint64_t acc[2] = {12345u, 1u}, racc[2] = {12345u, 1u}, hacc[2];
        double nsq = 0.0, rnsq = 0.0;
        int32_t rf = 0;
        const size_t ws = gs_unscale_check_sumsq_workspace_size(N, numel);
        void *dws = to_dev(NULL, ws);
        uint64_t *dacc = (uint64_t *)to_dev(acc, 16);
        double *dnsq = (double *)to_dev(&nsq, 8);
        HIPCHECK(hipMemset(dfound, 0, 4));
        check(gs_unscale_check_sumsq(N, dg, dout, numel, GS_F16, dS, dfound, dacc, dnsq, dws, ws,
                                     st) == GS_OK,
              "gs_unscale_check_sumsq returns GS_OK");
        orc_unscale_check_sumsq(N, (const uint16_t *const *)hg, ref, numel, S, &rf, racc, &rnsq);
        HIPCHECK(hipStreamSynchronize(st));
        from_dev(hacc, dacc, 16);
        from_dev(&nsq, dnsq, 8);
        check(hacc[0] == racc[0] && hacc[1] == racc[1], "128-bit sum of squares matches");
        check(memcmp(&nsq, &rnsq, 8) == 0, "norm squared matches");
        HIPCHECK(hipFree(dws));
        HIPCHECK(hipFree(dacc));
        HIPCHECK(hipFree(dnsq));
    }

    /* the hysteresis policy: overflow, overflow, clean */
    {
        float S2 = 1024.0f, hS2;
        int32_t t2 = 0, h2 = 2, f2 = 0, ht2, hh2;
        int64_t k2 = 0, hk2;
        float *dS2 = (float *)to_dev(&S2, 4);
        int32_t *dt2 = (int32_t *)to_dev(&t2, 4), *dh2 = (int32_t *)to_dev(&h2, 4);
        int32_t *df2 = (int32_t *)to_dev(&f2, 4);
        int64_t *dk2 = (int64_t *)to_dev(&k2, 8);
        const int32_t flags[3] = {1, 1, 0};
        for (int i = 0; i < 3; ++i) {
            f2 = flags[i];
            HIPCHECK(hipMemcpy(df2, &f2, 4, hipMemcpyHostToDevice));
            check(gs_update_scale_hysteresis(dS2, dt2, dh2, df2, 2.0f, 0.5f, 4, 2, 0, 1.0f, dk2,
                                             st) == GS_OK,
                  "gs_update_scale_hysteresis returns GS_OK");
            orc_update_scale_hysteresis(&S2, &t2, &h2, &f2, 2.0f, 0.5f, 4, 2, 0, 1.0f, &k2);
        }
        HIPCHECK(hipStreamSynchronize(st));
        from_dev(&hS2, dS2, 4);
        from_dev(&ht2, dt2, 4);
        from_dev(&hh2, dh2, 4);
        from_dev(&hk2, dk2, 8);
        check(hS2 == S2 && ht2 == t2 && hh2 == h2 && hk2 == k2 && S2 == 512.0f,
              "hysteresis state matches the oracle (the second overflow halves S)");
        HIPCHECK(hipFree(dS2));
        HIPCHECK(hipFree(dt2));
        HIPCHECK(hipFree(dh2));
        HIPCHECK(hipFree(df2));
        HIPCHECK(hipFree(dk2));
    }
    for (int t = 0; t < N; ++t) {
        HIPCHECK(hipFree((void *)dg[t]));
        HIPCHECK(hipFree(dout[t]));
        free(hg[t]);
        free(ho[t]);
        free(ref[t]);
    }
    HIPCHECK(hipFree(dS));
    HIPCHECK(hipFree(dtr));
    HIPCHECK(hipFree(dfound));
    HIPCHECK(hipFree(dskips));
}

/* ------------------------------------------------------------------- FP8 */
static uint16_t bf16_of(float f) {                /* RNE, for test inputs only */
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

static int64_t n_scales(int64_t rows, int64_t cols, int gran) {
    switch (gran) {
    case FP8_PER_TENSOR: return 1;
    case FP8_BLOCK_1x128: return rows * (cols / 128);
    case FP8_BLOCK_128x128: return (rows / 128) * (cols / 128);
    default: return rows * (cols / 32);
    }
}

static void test_quantize(hipStream_t st) {
    const int64_t R = 256, C = 512, n = R * C;
    uint16_t *hx = (uint16_t *)xmalloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) {
        const float u = ((float)(rnd() >> 8) + 0.5f) / 16777216.0f;
        const float v = ((float)(rnd() >> 8) + 0.5f) / 16777216.0f;
        float z = sqrtf(-2.0f * logf(u)) * cosf(6.2831853f * v);       /* N(0, 1) */
        z = ldexpf(z, (int)(rnd() % 24) - 12);
        hx[i] = bf16_of(z);
    }
    hx[17] = 0x7FC1u;                              /* a NaN and an Inf */
    hx[40000] = 0xFF80u;
    void *dx = to_dev(hx, (size_t)n * 2);
    uint8_t *dcodes = (uint8_t *)to_dev(NULL, (size_t)n);
    float *dsc = (float *)to_dev(NULL, (size_t)n / 32 * 4);
    float *dout = (float *)to_dev(NULL, (size_t)n * 4);
    uint16_t *dout16 = (uint16_t *)to_dev(NULL, (size_t)n * 2);
    int32_t *dnf = (int32_t *)to_dev(NULL, 4);
    const size_t ws = fp8_quantize_workspace_size(R, C, FP8_PER_TENSOR);
    void *dws = to_dev(NULL, ws);
    uint8_t *codes = (uint8_t *)xmalloc((size_t)n), *rcodes = (uint8_t *)xmalloc((size_t)n);
    float *sc = (float *)xmalloc((size_t)n / 32 * 4), *rsc = (float *)xmalloc((size_t)n / 32 * 4);
    float *out = (float *)xmalloc((size_t)n * 4), *rout = (float *)xmalloc((size_t)n * 4);
    uint16_t *out16 = (uint16_t *)xmalloc((size_t)n * 2), *rout16 = (uint16_t *)xmalloc((size_t)n * 2);
    const int grans[4] = {FP8_PER_TENSOR, FP8_BLOCK_1x128, FP8_BLOCK_128x128, FP8_BLOCK_1x32};
    char what[160];
    for (int fmt = 0; fmt < 2; ++fmt) {
        for (int gi = 0; gi < 4; ++gi) {
            const int g = grans[gi];
            const int64_t ns = n_scales(R, C, g);
            int32_t nf = 0, rnf = 0;
            HIPCHECK(hipMemset(dnf, 0, 4));
            const gs_status s = fp8_quantize(dx, GS_BF16, R, C, (fp8_format)fmt, (fp8_granularity)g,
                                             FP8_SCALE_FROM_AMAX, dcodes, dsc, dnf, dws, ws, st);
            const gs_status s2 = fp8_dequantize(dcodes, R, C, (fp8_format)fmt, (fp8_granularity)g,
                                                dsc, dout, st);
            const gs_status s3 = fp8_dequantize_bf16(dcodes, R, C, (fp8_format)fmt,
                                                     (fp8_granularity)g, dsc, dout16, st);
            orc_quantize(hx, GS_BF16, R, C, fmt, g, FP8_SCALE_FROM_AMAX, rcodes, rsc, &rnf);
            orc_dequantize(rcodes, R, C, fmt, g, rsc, rout);
            orc_dequantize_bf16(rcodes, R, C, fmt, g, rsc, rout16);
            HIPCHECK(hipStreamSynchronize(st));
            from_dev(codes, dcodes, (size_t)n);
            from_dev(sc, dsc, (size_t)ns * 4);
            from_dev(out, dout, (size_t)n * 4);
            from_dev(out16, dout16, (size_t)n * 2);
            from_dev(&nf, dnf, 4);
            snprintf(what, sizeof what, "fmt %d granularity %d: status, codes, scales, flag, "
                     "FP32 and BF16 dequantized values", fmt, g);
            check(s == GS_OK && s2 == GS_OK && s3 == GS_OK &&
                      memcmp(codes, rcodes, (size_t)n) == 0 &&
                      memcmp(sc, rsc, (size_t)ns * 4) == 0 && nf == rnf && nf == 1 &&
                      memcmp(out, rout, (size_t)n * 4) == 0 &&
                      memcmp(out16, rout16, (size_t)n * 2) == 0,
                  what);
        }
        /* per-tensor scaling without a workspace (the library's static scratch) */
        {
            int32_t nf = 0, rnf = 0;
            HIPCHECK(hipMemset(dnf, 0, 4));
            const gs_status s = fp8_quantize_no_workspace(dx, GS_BF16, R, C, (fp8_format)fmt,
                                                          FP8_PER_TENSOR, FP8_SCALE_FROM_AMAX,
                                                          dcodes, dsc, dnf, st);
            orc_quantize(hx, GS_BF16, R, C, fmt, FP8_PER_TENSOR, FP8_SCALE_FROM_AMAX, rcodes, rsc,
                         &rnf);
            HIPCHECK(hipStreamSynchronize(st));
            from_dev(codes, dcodes, (size_t)n);
            from_dev(sc, dsc, 4);
            from_dev(&nf, dnf, 4);
            snprintf(what, sizeof what, "fmt %d per-tensor without a workspace: codes, scale, flag",
                     fmt);
            check(s == GS_OK && memcmp(codes, rcodes, (size_t)n) == 0 && memcmp(sc, rsc, 4) == 0 &&
                      nf == rnf && nf == 1,
                  what);
        }
        /* MX blocks with E8M0 scale bytes */
        {
            uint8_t *dmx = (uint8_t *)dsc;         /* n / 32 bytes fit */
            uint8_t *mx = (uint8_t *)xmalloc((size_t)n / 32), *rmx = (uint8_t *)xmalloc((size_t)n / 32);
            int32_t rnf = 0;
            const gs_status s = fp8_quantize_mx(dx, GS_BF16, R, C, (fp8_format)fmt, dcodes, dmx,
                                                dnf, st);
            const gs_status s2 = fp8_dequantize_mx(dcodes, R, C, (fp8_format)fmt, dmx, dout, st);
            orc_quantize_mx(hx, GS_BF16, R, C, fmt, rcodes, rmx, &rnf);
            orc_dequantize_mx(rcodes, R, C, fmt, rmx, rout);
            HIPCHECK(hipStreamSynchronize(st));
            from_dev(codes, dcodes, (size_t)n);
            from_dev(mx, dmx, (size_t)n / 32);
            from_dev(out, dout, (size_t)n * 4);
            snprintf(what, sizeof what, "fmt %d MX 1x32: codes, E8M0 bytes, dequantized values", fmt);
            check(s == GS_OK && s2 == GS_OK && memcmp(codes, rcodes, (size_t)n) == 0 &&
                      memcmp(mx, rmx, (size_t)n / 32) == 0 &&
                      memcmp(out, rout, (size_t)n * 4) == 0,
                  what);
            free(mx);
            free(rmx);
        }
    }
    /* delayed scaling: three steps, the input doubling each step */
    {
        enum { H = 4 };
        float state = 1.0f, hist[H] = {0, 0, 0, 0}, used = 0.0f;
        float hstate, hhist[H], hused;
        int32_t pos = 0, hpos, rnf = 0;
        float *dstate = (float *)to_dev(&state, 4), *dhist = (float *)to_dev(hist, sizeof hist);
        float *dused = (float *)to_dev(&used, 4);
        int32_t *dpos = (int32_t *)to_dev(&pos, 4);
        for (int step = 0; step < 3; ++step) {
            if (step) {
                for (int64_t i = 0; i < n; ++i)
                    if ((hx[i] & 0x7F80u) != 0x7F80u && (hx[i] & 0x7F80u) < 0x7E80u && (hx[i] & 0x7F80u))
                        hx[i] = (uint16_t)(hx[i] + 0x80u);              /* x2: exponent + 1 */
                HIPCHECK(hipMemcpy(dx, hx, (size_t)n * 2, hipMemcpyHostToDevice));
            }
            const gs_status s = fp8_quantize_delayed(dx, GS_BF16, R, C, FP8_E4M3, dstate, dhist, H,
                                                     dpos, dcodes, dused, dnf, dws, ws, st);
            orc_quantize_delayed(hx, GS_BF16, R, C, FP8_E4M3, &state, hist, H, &pos, rcodes, &used,
                                 &rnf);
            HIPCHECK(hipStreamSynchronize(st));
            from_dev(codes, dcodes, (size_t)n);
            from_dev(&hstate, dstate, 4);
            from_dev(hhist, dhist, sizeof hhist);
            from_dev(&hused, dused, 4);
            from_dev(&hpos, dpos, 4);
            snprintf(what, sizeof what, "delayed step %d: codes, scale used, next scale, history, "
                     "position", step);
            check(s == GS_OK && memcmp(codes, rcodes, (size_t)n) == 0 &&
                      memcmp(&hused, &used, 4) == 0 && memcmp(&hstate, &state, 4) == 0 &&
                      memcmp(hhist, hist, sizeof hist) == 0 && hpos == pos,
                  what);
        }
        HIPCHECK(hipFree(dstate));
        HIPCHECK(hipFree(dhist));
        HIPCHECK(hipFree(dused));
        HIPCHECK(hipFree(dpos));
    }
    HIPCHECK(hipFree(dx));
    HIPCHECK(hipFree(dcodes));
    HIPCHECK(hipFree(dsc));
    HIPCHECK(hipFree(dout));
    HIPCHECK(hipFree(dout16));
    HIPCHECK(hipFree(dnf));
    HIPCHECK(hipFree(dws));
    free(hx);
    free(codes);
    free(rcodes);
    free(sc);
    free(rsc);
    free(out);
    free(rout);
    free(out16);
    free(rout16);
}

int main(void) {
    int ndev = 0;
    HIPCHECK(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        printf("no GPU\n");
        return 3;
    }
    HIPCHECK(hipSetDevice(0));
    hipStream_t st;
    HIPCHECK(hipStreamCreate(&st));
    test_unscale(st);
    test_quantize(st);
    HIPCHECK(hipStreamSynchronize(st));
    HIPCHECK(hipStreamDestroy(st));
    printf("%d failure(s)\n", failures);
    return failures != 0;
}
