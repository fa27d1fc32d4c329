/*
 * oracle.c -- plain, slow, obviously-correct CPU model of the loss-scaling and
 * FP8 scaled-cast path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may use it.  It shares no source, header,
 * table or helper with the HIP library: every number format is decoded and
 * encoded here from its definition, scalar by scalar, with no blocking,
 * fusion or reordering beyond what the pages describe.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 *        (no FTZ/DAZ: subnormal FP32 values are honoured everywhere).
 * All float arithmetic below is IEEE-754 binary32 with round-to-nearest-even
 * (x86-64 SSE; FLT_EVAL_METHOD == 0), which is what "fl32(.)" means in the
 * comments.  Exact intermediate values are carried in double where noted.
 *
 * Sources (the pages this follows; cited by page title and section):
 *   [LS]  "Loss scaling, FP8, and the failure that never crashes":
 *         section "Loss scaling, derived from the chain rule you already
 *         have" (the scaled-loss and recovered-gradient equations) and
 *         section "Worked example: a gradient that would have simply
 *         vanished" (the SimpleGradScaler listing and its 5-step trace).
 *   [NP]  "Numerical Precision, Mixed Precision, and Loss Scaling": the FP8
 *         specification paragraph (E4M3 bias 7 / max 448, E5M2 bias 15 /
 *         max 57344, E4M3 has no infinities and one NaN mantissa pattern),
 *         the FP16 range paragraph (65504, 2^-14, 2^-24) and the GradScaler
 *         defaults paragraph (65536, x2, x0.5, 2000).
 *   [WHY] "Why FP8 training is stable": section "How it works", Failure 1
 *         (one FP32 scale s per tensor; store x/s, multiply by s on the way
 *         out; s from the current max-abs) and "The seam" (1x128 tiles for
 *         activations, 128x128 blocks for weights).
 *   [MP]  "Mixed precision and FP8 training": section "FP8 training", the
 *         fp8_scaling.py listing (quant: divide, clamp to +-MAX, cast to FP8,
 *         cast back and multiply by the scale; per_tensor; per_block with the
 *         1e-12 floor on the block max-abs), and the hardware notes (MX
 *         formats: one scaling factor per 32 elements).
 *   [LS-d] "Loss Scaling" (glossary page), "Where it fits": loss scaling
 *         pairs with gradient clipping.
 *
 * Readings taken where the pages are silent (each is a definition here):
 *   - the unscale multiplies by inv = fl32(1/S) computed once;
 *   - the non-finite check looks at the FP32 outputs;
 *   - FP32 NaN outputs are written as the canonical quiet NaN 0x7FC00000;
 *   - block max-abs ignores NaN and +-Inf (finite-only amax);
 *   - the 1e-12 floor applies at every granularity;
 *   - a NaN input encodes as sign|0x7F, any other NaN quotient as 0x7F;
 *   - the sign of zero is kept (-0 and negative underflow give 0x80);
 *   - delayed scaling derives s from the maximum over the amax window;
 *   - the gradient norm is the exact sum of squares of the finite inputs;
 *   - the second scaler policy's knobs mean what their names say (budget
 *     of H overflows, refilled by clean steps or by growth; floor on S);
 *   - MX-style blocks are 1x32 along a row with a power-of-two (E8M0)
 *     scale, the smallest not below the pages' block scale.
 * Parity unpinned: these reading-defined rules (finite-only amax, NaN
 * canonicalisation, the floor at per-tensor granularity, the set-only flag
 * and the skip count) have no value on the pages to check against; they are
 * pinned only by rule-level unit tests of this file's own behaviour.  Every
 * function's finite-data behaviour is pinned externally (see the tests).
 * Partly unpinned for the same reason: the window maximum of delayed
 * scaling (pinned by its reduction to per-tensor scaling and the window's
 * closed form), the knob semantics of the second scaler policy (pinned by
 * its reduction to the GradScaler policy, closed forms and the page's two
 * comparisons), and the power-of-two rule of the MX scale (pinned by the
 * listing with that rule applied, the exponent-field identity and the
 * no-saturation property).
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Enumerations (same numeric values as the public ABI, restated here). */
enum { ORC_F16 = 1, ORC_BF16 = 2, ORC_F32 = 3 };
enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };
enum { ORC_PER_TENSOR = 0, ORC_BLOCK_1x128 = 1, ORC_BLOCK_128x128 = 2, ORC_BLOCK_1x32 = 3 };
enum { ORC_FROM_AMAX = 0, ORC_GIVEN = 1 };

/* ------------------------------------------------------------------ */
/* Bit-level helpers (memcpy: no aliasing games). */
static float f32_of_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static const uint32_t CANONICAL_NAN = 0x7FC00000u;

/* ------------------------------------------------------------------ */
/* FP16 (1 sign, 5 exponent bits with bias 15, 10 fraction bits) -> FP32.
 * [NP] FP16 range paragraph: max 65504, min normal 2^-14, min subnormal
 * 2^-24.  Value = (-1)^s * 2^(e-15) * (1 + m/1024) for 0<e<31,
 * (-1)^s * 2^-14 * m/1024 for e == 0, +-Inf / NaN for e == 31.
 * Every FP16 value is exactly representable in FP32, so the widening is
 * exact; it is computed in double and narrowed without rounding. */
float orc_f16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -14 - 10);
    else
        v = ldexp((double)(1024 + m), e - 15 - 10);
    return (float)(s ? -v : v);
}

/* BF16 is by definition the upper 16 bits of an FP32 word (1 sign,
 * 8 exponent bits, 7 fraction bits), so widening appends 16 zero bits. */
float orc_bf16_to_f32(uint16_t b) { return f32_of_bits((uint32_t)b << 16); }

/* ------------------------------------------------------------------ */
/* OCP FP8 formats, [NP] FP8 specification paragraph and [WHY] Failure 2:
 *   E4M3: 4 exponent bits, bias 7, 3 fraction bits, max normal 448,
 *         no infinities, NaN only as S.1111.111.
 *   E5M2: 5 exponent bits, bias 15, 2 fraction bits, max normal 57344,
 *         IEEE-style specials (exponent 31: Inf if fraction 0, else NaN). */
typedef struct { int ebits, mbits, bias; double maxval; } fp8_fmt;
static const fp8_fmt FMT[2] = {
    { 4, 3, 7, 448.0 },
    { 5, 2, 15, 57344.0 },
};

/* Exact value of an FP8 code (double holds it without rounding). */
double orc_fp8_decode(uint8_t code, int fmt)
{
    const fp8_fmt *F = &FMT[fmt];
    int s = code >> 7;
    int e = (code >> F->mbits) & ((1 << F->ebits) - 1);
    int m = code & ((1 << F->mbits) - 1);
    double v;
    if (fmt == ORC_E4M3 && e == 15 && m == 7)
        return s ? -NAN : NAN;
    if (fmt == ORC_E5M2 && e == 31) {
        if (m) return s ? -NAN : NAN;
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)
        v = ldexp((double)m, 1 - F->bias - F->mbits);
    else
        v = ldexp((double)((1 << F->mbits) + m), e - F->bias - F->mbits);
    return s ? -v : v;
}

/* Saturating round-to-nearest-even FP32 -> FP8 code, [MP] quant(): clamp
 * to [-MAX, MAX], then the cast rounds to the nearest FP8 value with ties
 * going to the code whose last fraction bit is 0.
 *   - NaN -> sign|0x7F (the only NaN pattern of E4M3; a quiet NaN of E5M2).
 *   - The sign is kept, also for zero results.
 *   - Procedure: a = min(|y|, MAX).  E = max(floor(log2 a), 1 - bias) is
 *     the binade (or the subnormal range).  The spacing of FP8 values there
 *     is q = 2^(E - mbits).  n = a / q rounded to the nearest integer, ties
 *     to even (a/q is exact: q is a power of two).  n*q is the result; it
 *     is assembled into exponent and fraction fields, with the carry into
 *     the next binade when n reaches 2^(mbits+1). */
uint8_t orc_fp8_encode(float y, int fmt)
{
    const fp8_fmt *F = &FMT[fmt];
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)y);
    if (a > F->maxval)
        a = F->maxval;                      /* saturation */
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);                     /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                          /* floor(log2 a) */
    int Emin = 1 - F->bias;
    if (E < Emin)
        E = Emin;
    double q = ldexp(1.0, E - F->mbits);
    double n = nearbyint(a / q);             /* default mode: ties to even */
    int N = (int)n;
    int one = 1 << F->mbits;                 /* implicit leading bit */
    int field_e, field_m;
    if (E == Emin && N < one) {              /* subnormal (or rounded to 0) */
        field_e = 0;
        field_m = N;
    } else {
        if (N == 2 * one) {                  /* rounded up into next binade */
            E += 1;
            N = one;
        }
        field_e = E + F->bias;
        field_m = N - one;
    }
    return (uint8_t)(sign | (field_e << F->mbits) | field_m);
}

/* ------------------------------------------------------------------ */
/* Fused unscale + non-finite check over a list of FP16 gradient tensors.
 * [LS] chain-rule section: the backward pass produced S*g; the recovered
 * gradient is g_scaled / S, formed in FP32.  [LS] SimpleGradScaler: any
 * Inf/NaN among the gradients means the step is skipped.
 *   inv = fl32(1/S) once; y = fl32(widen(g) * inv) per element;
 *   out = y, or the canonical NaN when y is NaN;
 *   *found_inf is set to 1 when any y is not finite, else left untouched. */
void orc_unscale_check(int32_t n, const uint16_t *const *grads,
                       float *const *outs, const int64_t *numels,
                       float S, int32_t *found_inf)
{
    float inv = 1.0f / S;
    int any = 0;
    for (int32_t t = 0; t < n; ++t) {
        const uint16_t *g = grads[t];
        float *o = outs[t];
        for (int64_t i = 0; i < numels[t]; ++i) {
            float y = orc_f16_to_f32(g[i]) * inv;
            if (!isfinite(y))
                any = 1;
            if (isnan(y))
                o[i] = f32_of_bits(CANONICAL_NAN);
            else
                o[i] = y;
        }
    }
    if (any)
        *found_inf = 1;
}

/* Unscale + check as orc_unscale_check, plus the sum of squares of the
 * gradients for norm clipping ("Loss Scaling", "Where it fits": loss scaling
 * pairs with gradient clipping; "Numerical Precision, Mixed Precision, and
 * Loss Scaling", the AMP sequence: unscale and inspect, then clip and update).
 * Exact definition: every finite FP16 value g is an integer multiple of
 * 2^-24 below 2^16 in magnitude, so G = |g| * 2^24 is an integer below 2^40
 * and X = sum G^2 over the finite inputs is an integer below 2^113 (for up
 * to 2^33 elements): it is accumulated exactly in 128 bits and ADDED to
 * sumsq[0] (low 64 bits) + sumsq[1] * 2^64.  The recovered-gradient norm
 * squared is then
 *   *norm_sq = fl64(fl64(X_total) * 2^-48) * fl64(inv * inv),
 * with fl64(X_total) the round-to-nearest-even conversion of the 128-bit
 * running total and inv = fl32(1/S) (inv * inv is exact in FP64); for a
 * power-of-two S this is the correctly rounded sum of y^2. */
void orc_unscale_check_sumsq(int32_t n, const uint16_t *const *grads,
                             float *const *outs, const int64_t *numels,
                             float S, int32_t *found_inf, uint64_t *sumsq,
                             double *norm_sq)
{
    orc_unscale_check(n, grads, outs, numels, S, found_inf);
    unsigned __int128 X = 0;
    for (int32_t t = 0; t < n; ++t)
        for (int64_t i = 0; i < numels[t]; ++i) {
            double g = (double)orc_f16_to_f32(grads[t][i]);
            if (!isfinite(g))
                continue;
            uint64_t G = (uint64_t)(fabs(g) * 16777216.0);   /* exact */
            X += (unsigned __int128)G * G;
        }
    unsigned __int128 total = ((unsigned __int128)sumsq[1] << 64) | sumsq[0];
    total += X;
    sumsq[0] = (uint64_t)total;
    sumsq[1] = (uint64_t)(total >> 64);
    float inv = 1.0f / S;
    double d = (double)total;                 /* round to nearest even */
    *norm_sq = (d * 0x1p-48) * ((double)inv * (double)inv);
}

/* Grow/backoff update of the loss scale, [LS] SimpleGradScaler.step with
 * [NP]'s GradScaler factors (backoff 0.5 instead of the listing's /2.0; the
 * two give the same FP32 result since both round the same exact value):
 *   overflow seen: S = fl32(S * backoff), tracker = 0, one more skip;
 *   clean step:    tracker += 1; when tracker >= interval,
 *                  S = fl32(S * growth) and tracker = 0.
 * The flag is consumed: *found_inf = 0 afterwards.  No clamp on S. */
void orc_update_scale(float *S, int32_t *tracker, int32_t *found_inf,
                      float growth, float backoff, int32_t interval,
                      int64_t *skips)
{
    if (*found_inf) {
        *S = *S * backoff;
        *tracker = 0;
        if (skips)
            *skips += 1;
    } else {
        *tracker += 1;
        if (*tracker >= interval) {
            *S = *S * growth;
            *tracker = 0;
        }
    }
    *found_inf = 0;
}

/* The second scaler policy of [NP]'s loss-scaler constants paragraph (the
 * DeepSpeed fp16 block): start 2^16, window 1000, hysteresis 2,
 * consecutive_hysteresis false, min_loss_scale 1.  The page names these
 * knobs without defining them; the plainest reading of each name:
 *   overflow step: skipped (skips += 1); the clean-step count restarts
 *                  (tracker = 0); if the hysteresis budget h is spent
 *                  (h <= 1) the scale is lowered,
 *                  S = max(fl32(S * backoff), min_scale),
 *                  otherwise one unit of budget is spent (h -= 1) and S
 *                  is kept;
 *   clean step:    with consecutive hysteresis the budget refills (h = H),
 *                  so only H overflows in a row lower S; then
 *                  tracker += 1 and when tracker >= window,
 *                  S = fl32(S * growth), tracker = 0 and, without
 *                  consecutive hysteresis, the budget refills there.
 *   The flag is consumed.  With H = 1 and min_scale = 0 this is exactly
 *   orc_update_scale (the GradScaler policy). */
void orc_update_scale_hysteresis(float *S, int32_t *tracker, int32_t *h,
                                 int32_t *found_inf, float growth, float backoff,
                                 int32_t window, int32_t H, int32_t consecutive,
                                 float min_scale, int64_t *skips)
{
    if (*found_inf) {
        if (skips)
            *skips += 1;
        *tracker = 0;
        if (*h <= 1) {
            float lowered = *S * backoff;
            *S = lowered > min_scale ? lowered : min_scale;
        } else {
            *h -= 1;
        }
    } else {
        if (consecutive)
            *h = H;
        *tracker += 1;
        if (*tracker >= window) {
            *S = *S * growth;
            *tracker = 0;
            if (!consecutive)
                *h = H;
        }
    }
    *found_inf = 0;
}

/* ------------------------------------------------------------------ */
/* FP8 scaled quantization, [MP] per_tensor / per_block / quant and [WHY]
 * Failure 1 and "The seam".  Input rows x cols row-major, BF16 or FP32,
 * widened exactly to FP32 first; everything after is FP32.
 * Blocks: per-tensor = the whole matrix; 1x128 = one row, 128 consecutive
 * columns; 128x128 = a square tile.  Scales are stored row-major, one per
 * block: [1], [rows][cols/128], [rows/128][cols/128]. */

static float load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == ORC_BF16)
        return orc_bf16_to_f32(((const uint16_t *)x)[idx]);
    return ((const float *)x)[idx];
}

static double fmt_max(int fmt) { return FMT[fmt].maxval; }

/* Largest finite |x| over a rectangular block (0 when it has none). */
float orc_block_amax(const void *x, int dtype, int64_t cols,
                     int64_t r0, int64_t nr, int64_t c0, int64_t nc)
{
    float amax = 0.0f;
    for (int64_t r = r0; r < r0 + nr; ++r)
        for (int64_t c = c0; c < c0 + nc; ++c) {
            float f = load_elem(x, dtype, r * cols + c);
            if (isfinite(f) && fabsf(f) > amax)
                amax = fabsf(f);
        }
    return amax;
}

/* s = fl32(max(amax, 1e-12) / MAX): the dequantization multiplier. */
float orc_scale_from_amax(float amax, int fmt)
{
    const float floor_ = 1e-12f;
    float a = amax > floor_ ? amax : floor_;
    return a / (float)fmt_max(fmt);
}

/* One element: y = fl32(f / s), clamp, RNE to FP8. */
uint8_t orc_cast(float f, float s, int fmt)
{
    if (isnan(f))
        return (uint8_t)((signbit(f) ? 0x80 : 0x00) | 0x7F);
    float y = f / s;
    if (isnan(y))
        return 0x7F;
    return orc_fp8_encode(y, fmt);
}

static void block_shape(int gran, int64_t rows, int64_t cols,
                        int64_t *br, int64_t *bc)
{
    if (gran == ORC_PER_TENSOR) { *br = rows; *bc = cols; }
    else if (gran == ORC_BLOCK_1x128) { *br = 1; *bc = 128; }
    else if (gran == ORC_BLOCK_1x32) { *br = 1; *bc = 32; }
    else { *br = 128; *bc = 128; }
}

/* Returns 0 on success, -1 when block granularity does not divide the
 * shape (the listing's reshape needs whole blocks). */
int orc_quantize(const void *x, int dtype, int64_t rows, int64_t cols,
                 int fmt, int gran, int mode, uint8_t *codes, float *scales,
                 int32_t *nonfinite)
{
    int64_t br, bc;
    block_shape(gran, rows, cols, &br, &bc);
    if (gran != ORC_PER_TENSOR && (rows % br != 0 || cols % bc != 0))
        return -1;
    int64_t nbr = (gran == ORC_PER_TENSOR) ? 1 : rows / br;
    int64_t nbc = (gran == ORC_PER_TENSOR) ? 1 : cols / bc;
    int any_nonfinite = 0;
    for (int64_t bi = 0; bi < nbr; ++bi)
        for (int64_t bj = 0; bj < nbc; ++bj) {
            int64_t r0 = bi * br, c0 = bj * bc;
            float s;
            if (mode == ORC_FROM_AMAX) {
                s = orc_scale_from_amax(
                    orc_block_amax(x, dtype, cols, r0, br, c0, bc), fmt);
                scales[bi * nbc + bj] = s;
            } else {
                s = scales[bi * nbc + bj];
            }
            for (int64_t r = r0; r < r0 + br; ++r)
                for (int64_t c = c0; c < c0 + bc; ++c) {
                    float f = load_elem(x, dtype, r * cols + c);
                    if (!isfinite(f))
                        any_nonfinite = 1;
                    codes[r * cols + c] = orc_cast(f, s, fmt);
                }
        }
    if (any_nonfinite && nonfinite)
        *nonfinite = 1;
    return 0;
}

/* Delayed per-tensor scaling, [WHY] Failure 1 (the scale comes from a short
 * history of recent max-abs values, so the scale applied this step reflects
 * earlier steps) and the [MP] "FP8 training" figure (per-tensor scaling
 * taken from recent amax values).  One step:
 *   1. codes = quant(x, s) with s = *scale_state (the given-scale cast:
 *      divide, clamp, round to nearest even);
 *   2. amax_t = largest finite |x| (0 if none);
 *   3. history[p] = amax_t with p = *pos mod H; *pos = (p + 1) mod H;
 *   4. *scale_state = fl32(max(max over the H history entries, 1e-12) / MAX),
 *      the scale for the next step.
 * Reading: the pages do not say how s follows from the history; it is taken
 * as the maximum over the window (the scale then covers every recent amax).  *scale_used receives the s of
 * step 1 (the dequantisation multiplier of these codes). */
int orc_quantize_delayed(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                         float *scale_state, float *history, int32_t hlen, int32_t *pos,
                         uint8_t *codes, float *scale_used, int32_t *nonfinite)
{
    if (hlen <= 0)
        return -1;
    const int32_t p = ((*pos % hlen) + hlen) % hlen;   /* position taken modulo H */
    const float s = *scale_state;
    if (orc_quantize(x, dtype, rows, cols, fmt, ORC_PER_TENSOR, ORC_GIVEN, codes,
                     scale_state, nonfinite) != 0)
        return -1;
    *scale_used = s;
    history[p] = orc_block_amax(x, dtype, cols, 0, rows, 0, cols);
    *pos = (p + 1) % hlen;
    float hmax = 0.0f;
    for (int32_t i = 0; i < hlen; ++i)
        if (history[i] > hmax)
            hmax = history[i];
    *scale_state = orc_scale_from_amax(hmax, fmt);
    return 0;
}

/* Dequantize, [MP] quant(): the FP8 value times its block's scale, in FP32.
 * out = fl32(decode(code) * s), canonical NaN for NaN results. */
int orc_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                   int gran, const float *scales, float *out)
{
    int64_t br, bc;
    block_shape(gran, rows, cols, &br, &bc);
    if (gran != ORC_PER_TENSOR && (rows % br != 0 || cols % bc != 0))
        return -1;
    int64_t nbc = (gran == ORC_PER_TENSOR) ? 1 : cols / bc;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t b = (gran == ORC_PER_TENSOR) ? 0 : (r / br) * nbc + c / bc;
            float v = (float)orc_fp8_decode(codes[r * cols + c], fmt);
            float o = v * scales[b];
            out[r * cols + c] = isnan(o) ? f32_of_bits(CANONICAL_NAN) : o;
        }
    return 0;
}

/* Dequantize to BF16: the FP32 result of orc_dequantize rounded once more,
 * to the nearest BF16 value with ties to an even last bit (the FP32 value
 * cast to the BF16 compute type); NaN -> 0x7FC0.  BF16 keeps FP32's sign and
 * exponent fields and the top 7 fraction bits, so the rounding acts on the
 * low 16 bits of the FP32 pattern: drop them, and add one unit when they are
 * above half a unit, or exactly half with the kept last bit odd (a carry
 * moves into the exponent, giving Inf past the largest BF16). */
static uint16_t bf16_rne(float y)
{
    if (isnan(y))
        return 0x7FC0;
    uint32_t b = bits_of_f32(y);
    uint32_t kept = b >> 16, dropped = b & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        ++kept;
    return (uint16_t)kept;
}

int orc_dequantize_bf16(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                        int gran, const float *scales, uint16_t *out)
{
    const int64_t n = rows * cols;
    float *f32 = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!f32)
        return -2;
    int rc = orc_dequantize(codes, rows, cols, fmt, gran, scales, f32);
    if (rc == 0)
        for (int64_t i = 0; i < n; ++i)
            out[i] = bf16_rne(f32[i]);
    free(f32);
    return rc;
}

/* MX-style blocks ("Mixed precision and FP8 training", hardware notes: MX
 * formats keep one scaling factor per 32 elements).  The pages do not say
 * how that factor is encoded; the reading here: blocks are 1x32 along a
 * row; the scale is a power of two stored as one E8M0 byte (2^(byte-127),
 * 0xFF = NaN), namely the smallest power of two not below the pages' own
 * block scale fl32(max(amax, 1e-12) / MAX), so that, as with that scale,
 * no finite element saturates; the cast is the same divide, clamp and
 * round-to-nearest-even.  Returns -1 when cols is not a multiple of 32. */
static float pow2_at_least(float s)           /* s positive, normal */
{
    int e;
    double m = frexp((double)s, &e);          /* s = m * 2^e, 0.5 <= m < 1 */
    return (float)(m == 0.5 ? ldexp(1.0, e - 1) : ldexp(1.0, e));
}

int orc_quantize_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt,
                    uint8_t *codes, uint8_t *scales_e8m0, int32_t *nonfinite)
{
    if (cols % 32 != 0)
        return -1;
    int any_nonfinite = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t bj = 0; bj < cols / 32; ++bj) {
            float s = pow2_at_least(orc_scale_from_amax(
                orc_block_amax(x, dtype, cols, r, 1, bj * 32, 32), fmt));
            int e;
            frexp((double)s, &e);
            scales_e8m0[r * (cols / 32) + bj] = (uint8_t)(e - 1 + 127);   /* s = 2^(e-1) */
            for (int64_t c = bj * 32; c < bj * 32 + 32; ++c) {
                float f = load_elem(x, dtype, r * cols + c);
                if (!isfinite(f))
                    any_nonfinite = 1;
                codes[r * cols + c] = orc_cast(f, s, fmt);
            }
        }
    if (any_nonfinite && nonfinite)
        *nonfinite = 1;
    return 0;
}

/* out = fl32(decode(code) * 2^(byte - 127)), canonical NaN; byte 0xFF is a
 * NaN scale. */
int orc_dequantize_mx(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                      const uint8_t *scales_e8m0, float *out)
{
    if (cols % 32 != 0)
        return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t b = scales_e8m0[r * (cols / 32) + c / 32];
            float s = b == 0xFF ? f32_of_bits(CANONICAL_NAN) : (float)ldexp(1.0, (int)b - 127);
            float v = (float)orc_fp8_decode(codes[r * cols + c], fmt);
            float o = v * s;
            out[r * cols + c] = isnan(o) ? f32_of_bits(CANONICAL_NAN) : o;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Array forms of the scalar codecs, for exhaustive checks from Python. */
void orc_fp8_encode_array(const float *y, int64_t n, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_fp8_encode(y[i], fmt);
}

void orc_cast_array(const float *f, int64_t n, float s, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_cast(f[i], s, fmt);
}

void orc_fp8_decode_table(int fmt, double *out256)
{
    for (int c = 0; c < 256; ++c)
        out256[c] = orc_fp8_decode((uint8_t)c, fmt);
}

void orc_f16_to_f32_array(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f32(h[i]);
}

uint32_t orc_canonical_nan_bits(void) { return CANONICAL_NAN; }
