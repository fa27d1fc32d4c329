/*
 * div_by_scale_sweep.c -- CPU check of the division the FP8 quantize kernels
 * use in place of one IEEE division per element.
 *
 * The cast divides each element by its block scale s ("Mixed precision and
 * FP8 training", section "FP8 training": quant divides, clamps to +-MAX and
 * casts).  The kernels instead form r = fl32(1/s) once per block and, per
 * element, q0 = fl32(|x| r), e = fma(-q0, s, |x|) (the exact remainder),
 * q = fma(e, r, q0): one Newton-style correction of the quotient (Markstein;
 * see Muller et al., "Handbook of Floating-Point Arithmetic", on division by
 * FMA).  The claim checked here, for s in the range the kernels use it,
 * 2^-80 <= s <= 2^126 (every scale derived from a block amax is inside it):
 *   - if the IEEE quotient fl32(|x| / s) is at least 2^-20, q equals it bit
 *     for bit (after the clamp to MAX that given scales get);
 *   - otherwise q is below 2^-17, half the smallest E5M2 subnormal (E4M3's
 *     is larger), so both round to the FP8 code 0.
 * So the FP8 code the kernels produce equals that of the IEEE quotient.
 *
 * Sweeps (per format, MAX = 448 and 57344):
 *   amax     random finite positive amax (uniform over bit patterns, so
 *            also below the 1e-12 floor), s = fl32(max(amax, fl32(1e-12)) /
 *            MAX), |x| uniform over the bit patterns in [0, amax];
 *   mid      quotients within +-8 ulps of every midpoint between adjacent
 *            positive FP8 values: x = fl32(m s) moved by k ulps, |x| <= amax,
 *            for random non-power-of-two amax;
 *   given    random s over the whole fast range and random finite |x|;
 *   gmid     the midpoint targeting with random given s.
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off (no FMA formed
 * from separate operations; fmaf is the fused operation v_fma_f32 performs).
 * Usage: div_by_scale_sweep [N_random] [--uncorrected]   (--uncorrected
 * drops the FMA correction, which must then fail: the check has teeth).
 * Prints one line per sweep and "mismatches TOTAL"; exit status 0 when the
 * result is the expected one.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f32(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t u32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint64_t next64(void)    /* splitmix64 (Steele, Lea, Flood 2014) */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static uint32_t below(uint32_t n) { return (uint32_t)(next64() % n); }

static int corrected = 1;

static float fast_div(float ax, float s, float r)
{
    const float q0 = ax * r;
    if (!corrected)
        return q0;
    const float e = fmaf(-q0, s, ax);
    return fmaf(e, r, q0);
}

/* one (|x|, s) pair: 1 when the claim holds */
static int check(float ax, float s, float maxv, int given)
{
    const float r = 1.0f / s;
    uint32_t qb = u32(fast_div(ax, s, r));
    uint32_t ib = u32(ax / s);
    if (given) {                          /* the kernels clamp a given scale's quotient */
        const uint32_t mb = u32(maxv);    /* unsigned min: NaN and Inf patterns give MAX */
        qb = qb < mb ? qb : mb;
        ib = ib < mb ? ib : mb;
    }
    if (f32(ib) >= 0x1p-20f)
        return qb == ib;
    return f32(qb) < 0x1p-17f;
}

static float amax_scale(float amax, float maxv)
{
    const float floor_ = f32(0x2B8CBCCCu);          /* fl32(1e-12) */
    return (amax > floor_ ? amax : floor_) / maxv;
}

/* positive FP8 midpoints (exact in double) of one format */
static int midpoints(int ebits, int mbits, int bias, double maxv, double *out)
{
    double prev = 0.0;
    int n = 0;
    for (int e = 0; e < (1 << ebits); ++e)
        for (int m = 0; m < (1 << mbits); ++m) {
            double v = e == 0 ? ldexp(m, 1 - bias - mbits) : ldexp((1 << mbits) + m, e - bias - mbits);
            if (v > maxv || (e == 0 && m == 0))
                continue;
            out[n++] = 0.5 * (prev + v);
            prev = v;
        }
    return n;
}

static float random_fast_scale(void)     /* 2^-80 <= s <= 2^126, any mantissa */
{
    const uint32_t lo = 0x17800000u, hi = 0x7E800000u;
    return f32(lo + below(hi - lo + 1));
}

int main(int argc, char **argv)
{
    long long nrand = 50000000;
    for (int i = 1; i < argc; ++i) {
        if (strcmp(argv[i], "--uncorrected") == 0)
            corrected = 0;
        else
            nrand = atoll(argv[i]);
    }
    const double maxs[2] = {448.0, 57344.0};
    const int eb[2] = {4, 5}, mb[2] = {3, 2}, bi[2] = {7, 15};
    long long total_bad = 0, total = 0;
    for (int f = 0; f < 2; ++f) {
        const float maxv = (float)maxs[f];
        long long bad = 0, cnt = 0;
        for (long long i = 0; i < nrand; ++i) {                 /* amax */
            const float amax = f32(1u + below(0x7F7FFFFFu));
            const float s = amax_scale(amax, maxv);
            const float ax = f32(below(u32(amax) + 1u));
            bad += !check(ax, s, maxv, 0);
            ++cnt;
        }
        printf("fmt %d amax: %lld pairs, %lld mismatches\n", f, cnt, bad);
        total_bad += bad; total += cnt;

        double mids[256];
        const int nm = midpoints(eb[f], mb[f], bi[f], maxs[f], mids);
        bad = cnt = 0;
        for (int j = 0; j < nm; ++j)                            /* mid */
            for (int t = 0; t < 20000; ++t) {
                uint32_t ab = 0x00800001u + below(0x7F000000u);  /* normal, random mantissa */
                if ((ab & 0x7FFFFFu) == 0)
                    ab |= 1u;                                    /* not a power of two */
                const float amax = f32(ab);
                const float s = amax_scale(amax, maxv);
                const float x0 = (float)(mids[j] * (double)s);
                if (!(x0 > 0.0f) || !isfinite(x0))
                    continue;
                for (int k = -8; k <= 8; ++k) {
                    const float ax = f32((uint32_t)((int64_t)u32(x0) + k));
                    if (!(ax > 0.0f) || ax > amax)
                        continue;
                    bad += !check(ax, s, maxv, 0);
                    ++cnt;
                }
            }
        printf("fmt %d mid: %d midpoints, %lld pairs, %lld mismatches\n", f, nm, cnt, bad);
        total_bad += bad; total += cnt;

        bad = cnt = 0;
        for (long long i = 0; i < nrand / 4; ++i) {             /* given */
            const float s = random_fast_scale();
            const float ax = f32(below(0x7F800000u));
            bad += !check(ax, s, maxv, 1);
            ++cnt;
        }
        printf("fmt %d given: %lld pairs, %lld mismatches\n", f, cnt, bad);
        total_bad += bad; total += cnt;

        bad = cnt = 0;
        for (int j = 0; j < nm; ++j)                            /* gmid */
            for (int t = 0; t < 5000; ++t) {
                const float s = random_fast_scale();
                const float x0 = (float)(mids[j] * (double)s);
                if (!(x0 > 0.0f) || !isfinite(x0))
                    continue;
                for (int k = -8; k <= 8; ++k) {
                    const float ax = f32((uint32_t)((int64_t)u32(x0) + k));
                    if (!(ax > 0.0f) || !isfinite(ax))
                        continue;
                    bad += !check(ax, s, maxv, 1);
                    ++cnt;
                }
            }
        printf("fmt %d gmid: %lld pairs, %lld mismatches\n", f, cnt, bad);
        total_bad += bad; total += cnt;
    }
    printf("pairs %lld\nmismatches %lld\n", total, total_bad);
    return corrected ? (total_bad != 0) : (total_bad == 0);
}
