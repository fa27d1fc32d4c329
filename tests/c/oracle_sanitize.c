/* Every entry point of the oracle (oracle/oracle.c) run on exactly sized
 * heap buffers, for a build with -fsanitize=address,undefined
 * -fno-sanitize-recover=all: an out-of-bounds access, a use of freed or
 * uninitialised-size memory, a signed overflow or any other undefined
 * behaviour aborts the run.  Inputs are seeded bit patterns (special values
 * included), edge sizes (empty tensors, ragged tails, single elements) and
 * degenerate given scales.  Prints "done" and exits 0 when every call
 * returned as documented. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's functions (oracle/oracle.c) */
float orc_f16_to_f32(uint16_t h);
float orc_bf16_to_f32(uint16_t b);
double orc_fp8_decode(uint8_t code, int fmt);
uint8_t orc_fp8_encode(float y, int fmt);
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
float orc_block_amax(const void *x, int dtype, int64_t cols, int64_t r0, int64_t nr,
                     int64_t c0, int64_t nc);
float orc_scale_from_amax(float amax, int fmt);
uint8_t orc_cast(float f, float s, int fmt);
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
void orc_fp8_encode_array(const float *y, int64_t n, int fmt, uint8_t *out);
void orc_cast_array(const float *f, int64_t n, float s, int fmt, uint8_t *out);
void orc_fp8_decode_table(int fmt, double *out256);
void orc_f16_to_f32_array(const uint16_t *h, int64_t n, float *out);
uint32_t orc_canonical_nan_bits(void);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {                       /* xorshift64*, test inputs only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int failures = 0;
static void expect(int ok, const char *what) {
    if (!ok) {
        printf("FAIL %s\n", what);
        ++failures;
    }
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        printf("out of memory\n");
        exit(2);
    }
    return p;
}

/* n elements of the given dtype (2 = BF16 bits, 3 = FP32), 1/16 special */
static void *make_input(int dtype, int64_t n) {
    const size_t es = dtype == 2 ? 2 : 4;
    uint8_t *p = (uint8_t *)xmalloc((size_t)n * es);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = rnd();
        const uint32_t k = rnd() & 15;
        if (k == 0) b = (rnd() & 1) ? 0x7FC00001u : 0xFF800000u;      /* NaN, -Inf */
        else if (k == 1) b = (rnd() & 1) ? 0x00000000u : 0x80000000u; /* +-0 */
        else b = (b & 0x80000000u) | ((0x30000000u + (b & 0x1FFFFFFFu)) & 0x7FFFFFFFu);
        if (dtype == 2) {
            const uint16_t h = (uint16_t)(b >> 16);
            memcpy(p + (size_t)i * 2, &h, 2);
        } else {
            memcpy(p + (size_t)i * 4, &b, 4);
        }
    }
    return p;
}

static void test_codecs(void) {
    double table[256];
    for (int fmt = 0; fmt < 2; ++fmt) {
        orc_fp8_decode_table(fmt, table);
        for (int c = 0; c < 256; ++c) {
            expect(table[c] == table[c] || isnan(orc_fp8_decode((uint8_t)c, fmt)), "decode table");
            if (!isnan(table[c]) && !isinf(table[c]))
                expect(orc_fp8_encode((float)table[c], fmt) == (uint8_t)c ||
                       table[c] == 0.0, "encode(decode(c)) == c");
        }
        float y[1000];
        uint8_t o[1000];
        for (int i = 0; i < 1000; ++i) {
            const uint32_t b = rnd();
            memcpy(&y[i], &b, 4);
        }
        orc_fp8_encode_array(y, 1000, fmt, o);
        orc_cast_array(y, 1000, 0.75f, fmt, o);
        (void)orc_cast(y[3], 0.0f, fmt);
        (void)orc_scale_from_amax(0.0f, fmt);
    }
    uint16_t h[777];
    float f[777];
    for (int i = 0; i < 777; ++i) h[i] = (uint16_t)rnd();
    orc_f16_to_f32_array(h, 777, f);
    expect(orc_canonical_nan_bits() == 0x7FC00000u, "canonical NaN");
    (void)orc_bf16_to_f32(0x7F80u);
    (void)orc_f16_to_f32(0x0001u);
}

static void test_unscale(void) {
    const int64_t sizes[6] = {0, 1, 7, 2048, 2049, 5000};
    uint16_t *g[6];
    float *o[6];
    for (int t = 0; t < 6; ++t) {
        g[t] = (uint16_t *)xmalloc((size_t)sizes[t] * 2);
        o[t] = (float *)xmalloc((size_t)sizes[t] * 4);
        for (int64_t i = 0; i < sizes[t]; ++i) g[t][i] = (uint16_t)rnd();
    }
    int32_t found = 0;
    orc_unscale_check(6, (const uint16_t *const *)g, o, sizes, 65536.0f, &found);
    expect(found == 1, "random FP16 patterns include Inf/NaN");
    uint64_t acc[2] = {0, 0};
    double norm = 0.0;
    found = 0;
    orc_unscale_check_sumsq(6, (const uint16_t *const *)g, o, sizes, 3.0f, &found, acc, &norm);
    orc_unscale_check(0, NULL, NULL, NULL, 1.0f, &found);
    for (int t = 0; t < 6; ++t) {
        free(g[t]);
        free(o[t]);
    }
    float S = 65536.0f;
    int32_t tracker = 0, flag = 0, h = 2;
    int64_t skips = 0;
    for (int k = 0; k < 5000; ++k) {
        flag = (rnd() % 50) == 0;
        orc_update_scale(&S, &tracker, &flag, 2.0f, 0.5f, 7, &skips);
    }
    S = 65536.0f;
    tracker = 0;
    for (int k = 0; k < 5000; ++k) {
        flag = (rnd() % 20) == 0;
        orc_update_scale_hysteresis(&S, &tracker, &h, &flag, 2.0f, 0.5f, 13, 2, (int32_t)(k & 1),
                                    1.0f, 0.5f > 0 ? &skips : NULL);
    }
    orc_update_scale(&S, &tracker, &flag, 2.0f, 0.5f, 3, NULL);
}

static int64_t n_scales(int64_t rows, int64_t cols, int gran) {
    switch (gran) {
    case 0: return 1;
    case 1: return rows * (cols / 128);
    case 2: return (rows / 128) * (cols / 128);
    default: return rows * (cols / 32);
    }
}

static void test_quantize(void) {
    const int64_t shapes[4][2] = {{37, 53}, {3, 256}, {256, 384}, {5, 96}};
    for (int dtype = 2; dtype <= 3; ++dtype)
        for (int gran = 0; gran < 4; ++gran)
            for (int fmt = 0; fmt < 2; ++fmt)
                for (int mode = 0; mode < 2; ++mode) {
                    const int64_t r = shapes[gran][0], c = shapes[gran][1], n = r * c;
                    const int64_t ns = n_scales(r, c, gran);
                    void *x = make_input(dtype, n);
                    uint8_t *codes = (uint8_t *)xmalloc((size_t)n);
                    float *sc = (float *)xmalloc((size_t)ns * 4);
                    float *out = (float *)xmalloc((size_t)n * 4);
                    for (int64_t i = 0; i < ns; ++i) {
                        const uint32_t k = rnd() % 8;
                        sc[i] = k == 0 ? 0.0f : k == 1 ? INFINITY : k == 2 ? NAN
                              : k == 3 ? -2.0f : k == 4 ? 1e-40f : ldexpf(1.0f, (int)(rnd() % 60) - 30);
                    }
                    int32_t nf = 0;
                    expect(orc_quantize(x, dtype, r, c, fmt, gran, mode, codes, sc, &nf) == 0,
                           "quantize returns 0");
                    expect(orc_dequantize(codes, r, c, fmt, gran, sc, out) == 0, "dequantize returns 0");
                    uint16_t *out16 = (uint16_t *)xmalloc((size_t)n * 2);
                    expect(orc_dequantize_bf16(codes, r, c, fmt, gran, sc, out16) == 0,
                           "bf16 dequantize returns 0");
                    for (int64_t i = 0; i < n; ++i) {
                        uint32_t b;
                        memcpy(&b, &out[i], 4);
                        if (isnan(out[i])) expect(out16[i] == 0x7FC0u, "bf16 NaN is canonical");
                        else if ((b & 0xFFFFu) == 0) expect(out16[i] == (uint16_t)(b >> 16), "exact bf16 kept");
                    }
                    free(out16);
                    if (gran == 3 && mode == 0) {
                        uint8_t *e8 = (uint8_t *)xmalloc((size_t)ns);
                        expect(orc_quantize_mx(x, dtype, r, c, fmt, codes, e8, &nf) == 0, "mx quantize");
                        expect(orc_dequantize_mx(codes, r, c, fmt, e8, out) == 0, "mx dequantize");
                        free(e8);
                    }
                    if (gran == 0 && mode == 0) {
                        float state = 1.0f, used = 0.0f, hist[4] = {0, 0, 0, 0};
                        int32_t pos = 0;
                        for (int step = 0; step < 6; ++step)
                            expect(orc_quantize_delayed(x, dtype, r, c, fmt, &state, hist, 4, &pos,
                                                        codes, &used, &nf) == 0, "delayed quantize");
                    }
                    if (n > 0) (void)orc_block_amax(x, dtype, c, 0, r, 0, c);
                    free(x);
                    free(codes);
                    free(sc);
                    free(out);
                }
    /* empty matrix, per-tensor: the scale is still written */
    float s0 = -1.0f;
    int32_t nf = 0;
    uint8_t dummy = 0;
    expect(orc_quantize(&dummy, 2, 0, 5, 0, 0, 0, &dummy, &s0, &nf) == 0 && s0 > 0.0f,
           "empty per-tensor writes the floor scale");
}

int main(void) {
    test_codecs();
    test_unscale();
    test_quantize();
    printf("%d failure(s)\ndone\n", failures);
    return failures != 0;
}
