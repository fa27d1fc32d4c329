/*
 * gs.h -- C ABI of libgsfp8: dynamic loss scaling and FP8 scaled casting on
 * AMD MI355X (gfx950).
 *
 * Every entry point takes plain pointers and sizes.  Pointers documented as
 * "device" are HIP device allocations on the current device; "host" pointers
 * are read during the call only.  All work is enqueued on `stream` (a
 * hipStream_t; NULL means the null stream), asynchronously: no call
 * synchronises the host, reads device memory from the host, or allocates on
 * a repeated call with the same arguments.  Device buffers must stay alive
 * until the enqueued work has finished.  The one exception is the first
 * call of gs_unscale_check / gs_unscale_check_sumsq with a new gradient
 * list: it takes device memory for the list's chunk descriptors and uploads
 * them on an internal stream, waiting for that upload only; repeated calls
 * with the same list do neither.  After that first call every entry point
 * can be captured in a HIP graph: none allocates, copies from the host or
 * records a memset.
 *
 * Descriptor lifetime: the library caches the descriptors of at most 64
 * lists / 1 GiB and evicts the least recently used list when a new one does
 * not fit.  Eviction never frees memory or waits for the device: the
 * evicted buffer is reused for a later list once every kernel that read it
 * has finished (tracked by an event per stream).  A list used by a call
 * made while its stream was capturing a graph is never evicted, so a
 * captured graph may be replayed at any later time; such lists stay cached
 * until the process ends.  Idle retired buffers beyond 1 GiB per device are
 * freed (hipFree, which synchronises the device), which happens only when
 * callers keep creating lists larger than every retired one.
 *
 * Threads: entry points may be called from several host threads at once
 * (each on its own stream, or the same one).  The descriptor cache is
 * locked, and an unscale call enqueues its kernel while holding that lock,
 * so no thread's eviction can retire a list between another thread's lookup
 * and its launch.  Another thread may capture a graph meanwhile when its
 * capture mode permits this thread's first call with a new list (HIP's
 * thread-local or relaxed capture modes), since that call allocates and
 * synchronises its own upload stream.  Calls whose device outputs or
 * workspaces overlap must be ordered by the caller (streams or events), as
 * for any asynchronous work.
 *
 * Errors: argument errors are detected on the host and returned before
 * anything is enqueued, with no side effects.  Non-finite DATA is never an
 * error; it is reported through the found_inf / nonfinite flags.  A failing
 * HIP call returns GS_ERR_HIP.
 *
 * Sources (cited by page title and section):
 *   "Loss scaling, FP8, and the failure that never crashes" -- section
 *     "Loss scaling, derived from the chain rule you already have" (scaled
 *     loss S*L gives scaled gradients S*g; recovered gradient g_scaled / S in
 *     FP32; skip and halve on Inf/NaN, double after a run of clean steps) and
 *     the SimpleGradScaler listing of the worked-example section.
 *   "Numerical Precision, Mixed Precision, and Loss Scaling" -- the FP8
 *     specification paragraph (OCP E4M3 / E5M2), the FP16 range paragraph,
 *     the GradScaler defaults paragraph (65536, x2.0, x0.5, 2000) and the
 *     six-step AMP sequence (unscale and inspect; skip invalid steps;
 *     adjust the scale).
 *   "Why FP8 training is stable" -- "How it works", Failure 1 (one FP32 s:
 *     store x/s, multiply by s on the way out; s from the current max-abs)
 *     and "The seam" (1x128 activation tiles, 128x128 weight blocks).
 *   "Mixed precision and FP8 training" -- section "FP8 training",
 *     fp8_scaling.py (quant, per_tensor, per_block with the 1e-12 floor),
 *     and the hardware notes (MX formats: one scale per 32 elements).
 */
#ifndef GS_FP8_H
#define GS_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gs_status;
#define GS_OK             0
#define GS_ERR_NULL      -1  /* a required pointer is NULL                          */
#define GS_ERR_SIZE      -2  /* negative count or size, or too large                */
#define GS_ERR_SHAPE     -3  /* block granularity does not divide rows x cols        */
#define GS_ERR_DTYPE     -4  /* unsupported element type for this call               */
#define GS_ERR_ARG       -5  /* bad enum value, factor or interval                   */
#define GS_ERR_ALIGN     -6  /* pointer not aligned to its element size              */
#define GS_ERR_WORKSPACE -7  /* workspace missing or smaller than required           */
#define GS_ERR_HIP       -8  /* a HIP runtime call or kernel launch failed           */

typedef enum { GS_F16 = 1, GS_BF16 = 2, GS_F32 = 3 } gs_dtype;
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format;
typedef enum {
    FP8_PER_TENSOR = 0, FP8_BLOCK_1x128 = 1, FP8_BLOCK_128x128 = 2, FP8_BLOCK_1x32 = 3
} fp8_granularity;
typedef enum { FP8_SCALE_FROM_AMAX = 0, FP8_SCALE_GIVEN = 1 } fp8_scale_mode;

/*
 * gs_unscale_check -- fused multi-tensor unscale + non-finite check.
 * "Loss scaling, FP8, and the failure that never crashes": the recovered
 * gradient is g_scaled / S, computed in FP32 before the optimizer; any Inf or
 * NaN means the step must be skipped.  Here: inv = fl32(1/S) once, then for
 * every element y = fl32(fp32(g) * inv); the output is y, or the canonical
 * quiet NaN 0x7FC00000 when y is NaN; *found_inf is set to 1 when any y is
 * not finite.  The whole list is processed by one kernel launch.
 *
 *   n          number of tensors (>= 0).
 *   grads      host array of n device pointers to FP16 gradients (2-byte
 *              aligned; 16-byte alignment takes the vector path).
 *   outs       host array of n device pointers to FP32 outputs (4-byte
 *              aligned), each with room for numels[i] floats; an output must
 *              not overlap any input or other output.
 *   numels     host array of n element counts (>= 0; 0 is allowed).
 *   in_dtype   must be GS_F16.
 *   scale      device pointer to the current loss scale S (FP32), read only.
 *   found_inf  device int32, only ever written with 1 (set-only: the caller
 *              zeroes it once per step, several calls may OR into it, and
 *              gs_update_scale consumes and clears it).
 *   stream     hipStream_t.
 * The list is cut into 2048-element chunks whose descriptors (addresses and
 * sizes) are built on the first call with a given (grads, outs, numels) list
 * and cached on the device (lifetime rules at the top of this file), so a
 * repeated call with the same list uploads nothing.  That first call
 * uploads synchronously (the upload has finished when the call returns).
 * Device addresses must lie below 2^48 (GS_ERR_ARG otherwise; every current
 * AMD GPU address does).
 */
gs_status gs_unscale_check(int32_t n, const void *const *grads, float *const *outs,
                           const int64_t *numels, gs_dtype in_dtype, const float *scale,
                           int32_t *found_inf, void *stream);

/*
 * gs_unscale_list_descriptors -- the chunk descriptors gs_unscale_check
 * builds for this gradient list, written to host memory (for inspection and
 * tests; no HIP call, nothing on the device).  Chunk k of the list (tensors
 * in order, empty ones contribute none, each cut into 2048-element chunks,
 * its last chunk ragged) is two words:
 *   desc_out[2k]     = address of the chunk's first FP16 input element
 *                      | (element count << 48 when the chunk is ragged, else 0)
 *   desc_out[2k + 1] = address of the chunk's first FP32 output element
 *                      | 1 when the tensor's input or output address is not
 *                      16-byte aligned (the element-wise path), else 0
 *   grads, outs, numels  as gs_unscale_check (host arrays; the addresses are
 *                        not dereferenced).
 *   desc_out   host array of 2 * capacity words, or NULL to count only.
 * Returns the number of chunks (>= 0), or a negative gs_status: argument
 * errors as gs_unscale_check, GS_ERR_ARG when an address reaches 2^48,
 * GS_ERR_SIZE when capacity is smaller than the count.
 */
int64_t gs_unscale_list_descriptors(int32_t n, const void *const *grads, float *const *outs,
                                    const int64_t *numels, uint64_t *desc_out, int64_t capacity);

/*
 * gs_unscale_check_sumsq_workspace_size -- bytes of device workspace
 * gs_unscale_check_sumsq needs for a list with these element counts:
 * 16 * (sum over tensors of ceil(numels[i] / 2048) + 1024).  Returns 0 for
 * invalid counts (n < 0, a negative count, numels NULL with n > 0).
 */
size_t gs_unscale_check_sumsq_workspace_size(int32_t n, const int64_t *numels);

/*
 * gs_unscale_check_sumsq -- gs_unscale_check plus the exact sum of squares
 * of the gradients, for norm clipping.  The AMP step sequence of "Numerical
 * Precision, Mixed Precision, and Loss Scaling" unscales and inspects the
 * gradients, then clips them before the update, and "Loss Scaling" (section
 * "Where it fits") pairs loss scaling with gradient clipping; clipping by
 * global norm needs the norm of the recovered gradients, computed here in the
 * same pass over the FP16 data.
 * Outputs and found_inf exactly as gs_unscale_check.  In addition:
 *   X = sum over the FINITE inputs g of (|g| * 2^24)^2, an exact integer
 *       (every finite FP16 value is a multiple of 2^-24 below 2^16);
 *   sumsq[0] + sumsq[1] * 2^64 += X (128-bit running total, device uint64
 *       [2], 8-byte aligned; the caller zeroes it once per step, so several
 *       calls, e.g. one per gradient bucket, accumulate);
 *   *norm_sq = fl64(fl64(total) * 2^-48) * (inv * inv), with fl64(total)
 *       the round-to-nearest-even FP64 value of the new running total and
 *       inv = fl32(1/S) widened to FP64 (device double, 8-byte aligned).
 *       For a power-of-two S this is the correctly rounded sum of y^2 over
 *       the finite outputs; it does not depend on the launch configuration.
 *   Inf and NaN inputs are left out of X (they set found_inf; such a step
 *   is skipped anyway).
 *   workspace: device buffer of at least
 *       gs_unscale_check_sumsq_workspace_size(n, numels) bytes, 16-byte
 *       aligned, scratch (no initialisation needed).
 * Other arguments, the descriptor cache and errors as gs_unscale_check.
 * An empty list still updates *norm_sq from the running total.  Three
 * launches on `stream` (the unscale pass writing one partial per chunk, a
 * second-level reduction, a one-workgroup final add); no host
 * synchronisation.
 */
gs_status gs_unscale_check_sumsq(int32_t n, const void *const *grads, float *const *outs,
                                 const int64_t *numels, gs_dtype in_dtype, const float *scale,
                                 int32_t *found_inf, uint64_t *sumsq, double *norm_sq,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * gs_update_scale -- grow/backoff/skip state machine, kept on the device.
 * SimpleGradScaler.step ("Loss scaling, FP8, and the failure that never
 * crashes", worked example) with the GradScaler defaults paragraph of
 * "Numerical Precision, Mixed Precision, and Loss Scaling":
 *   if *found_inf != 0:  S = fl32(S * backoff_factor); *growth_tracker = 0;
 *                        *skip_count += 1 (when skip_count is not NULL)
 *   else:                *growth_tracker += 1; if it reaches growth_interval,
 *                        S = fl32(S * growth_factor) and *growth_tracker = 0
 *   then *found_inf = 0.  No floor or ceiling: S may reach 0 or +Inf.
 *
 *   scale, growth_tracker, found_inf: device scalars (FP32, int32, int32).
 *   growth_factor, backoff_factor: finite and > 0 (defaults 2.0, 0.5).
 *   growth_interval: > 0 (default 2000).
 *   skip_count: device int64 or NULL.
 * One single-lane kernel on `stream`; no host synchronisation.
 */
gs_status gs_update_scale(float *scale, int32_t *growth_tracker, int32_t *found_inf,
                          float growth_factor, float backoff_factor, int32_t growth_interval,
                          int64_t *skip_count, void *stream);

/*
 * gs_update_scale_hysteresis -- the second loss-scaler policy of "Numerical
 * Precision, Mixed Precision, and Loss Scaling" (loss-scaler constants
 * paragraph: the DeepSpeed fp16 block, start 2^16, loss_scale_window 1000,
 * hysteresis 2, consecutive_hysteresis false, min_loss_scale 1).  The page
 * names the knobs; their meaning here is the plain reading of the names:
 *   if *found_inf != 0:  *skip_count += 1 (when not NULL); *growth_tracker = 0;
 *                        if *hysteresis_left <= 1:
 *                            S = max(fl32(S * backoff_factor), min_scale)
 *                        else *hysteresis_left -= 1 (S kept)
 *   else:                if consecutive_hysteresis, *hysteresis_left = hysteresis;
 *                        *growth_tracker += 1; when it reaches growth_interval,
 *                        S = fl32(S * growth_factor), *growth_tracker = 0 and,
 *                        if not consecutive_hysteresis,
 *                        *hysteresis_left = hysteresis
 *   then *found_inf = 0.
 * So an overflow always skips the step, but S is lowered only on the
 * hysteresis-th overflow since the budget was last refilled (only
 * consecutive ones count when consecutive_hysteresis is 1), and never below
 * min_scale.  With hysteresis 1 and min_scale 0 this is gs_update_scale.
 *
 *   scale, growth_tracker, hysteresis_left, found_inf: device scalars
 *       (FP32, int32, int32, int32); start hysteresis_left at `hysteresis`.
 *   growth_factor, backoff_factor: finite and > 0 (2.0, 0.5).
 *   growth_interval: > 0 (the window, 1000).  hysteresis: >= 1 (2).
 *   consecutive_hysteresis: 0 or 1 (0).  min_scale: finite, >= 0 (1.0).
 *   skip_count: device int64 or NULL.
 * One single-lane kernel on `stream`; no host synchronisation.
 */
gs_status gs_update_scale_hysteresis(float *scale, int32_t *growth_tracker,
                                     int32_t *hysteresis_left, int32_t *found_inf,
                                     float growth_factor, float backoff_factor,
                                     int32_t growth_interval, int32_t hysteresis,
                                     int32_t consecutive_hysteresis, float min_scale,
                                     int64_t *skip_count, void *stream);

/*
 * fp8_quantize_workspace_size -- bytes of device workspace fp8_quantize
 * needs for this shape and granularity in FP8_SCALE_FROM_AMAX mode: 32 KiB of
 * per-workgroup partial maxima for per-tensor scaling (the scale depends on
 * the whole tensor: one pass writes the partial maxima, then the cast pass
 * derives the scale from them -- every cast workgroup itself for a tensor of
 * at most 192 MiB, one extra workgroup beforehand for a larger one); block
 * granularities need none.  Returns 0 when no workspace is needed.
 */
size_t fp8_quantize_workspace_size(int64_t rows, int64_t cols, fp8_granularity g);

/*
 * fp8_quantize -- scaled, saturating, round-to-nearest-even cast to OCP FP8.
 * fp8_scaling.py in "Mixed precision and FP8 training" (quant, per_tensor,
 * per_block) and Failure 1 / "The seam" of "Why FP8 training is stable".
 * The input is widened exactly to FP32; per block:
 *   FROM_AMAX: amax = largest finite |x| in the block (0 if none);
 *              s = fl32(max(amax, fl32(1e-12)) / MAX), written to scales.
 *   GIVEN:     s = scales[block] (read).
 *   code = NaN x  -> sign|0x7F;
 *          else y = fl32(x / s) (IEEE division); NaN y -> 0x7F;
 *          else clamp y to [-MAX, MAX] and round to the nearest FP8 value,
 *          ties to an even last fraction bit, keeping the sign (also of 0).
 *   MAX = 448 (E4M3) or 57344 (E5M2).  Dequantisation is decode(code) * s.
 *
 *   x          device, row-major rows x cols, GS_BF16 or GS_F32, 16-byte
 *              aligned (GS_ERR_ALIGN otherwise).
 *   rows, cols >= 0.  FP8_BLOCK_1x128 needs cols % 128 == 0;
 *              FP8_BLOCK_1x32 needs cols % 32 == 0;
 *              FP8_BLOCK_128x128 needs rows % 128 == 0 and cols % 128 == 0
 *              (GS_ERR_SHAPE otherwise).  Per-tensor takes any shape.
 *   codes      device uint8, rows x cols row-major, 16-byte aligned (1x128
 *              and 1x32 blocks run along the contiguous dimension).
 *   scales     device FP32, one per block, row-major: [1] (per-tensor),
 *              [rows][cols/128] (1x128), [rows][cols/32] (1x32) or
 *              [rows/128][cols/128] (128x128).
 *              Written in FROM_AMAX mode, read in GIVEN mode.  A per-tensor
 *              quantize of an empty matrix still writes scales[0].
 *   nonfinite  device int32 or NULL; set to 1 when any input is NaN or Inf
 *              (set-only, never cleared).
 *   workspace  device buffer of at least fp8_quantize_workspace_size()
 *              bytes (may be NULL when that is 0); contents need no
 *              initialisation and are scratch.
 *   stream     hipStream_t.
 */
gs_status fp8_quantize(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                       fp8_format fmt, fp8_granularity g, fp8_scale_mode mode,
                       uint8_t *codes, float *scales, int32_t *nonfinite,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp8_quantize_no_workspace -- fp8_quantize for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments minus the workspace,
 * the same results bit for bit.  Per-tensor scaling from the amax keeps its
 * partial maxima (at most 8192 words) in a static 32 KiB device array of the
 * library instead of a caller workspace; every other granularity and mode
 * needs no scratch memory at all.  The call allocates nothing.
 *   - Each GPU holds its own copy of the array until the process ends; the
 *     first call on a device looks up its address (do that first call
 *     outside graph capture).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind (nothing in it needs clearing: each call writes the partials it
 *     reads).  Per-tensor FROM_AMAX calls that may run at the same time on
 *     one GPU (different streams without ordering) race on the array and
 *     must be ordered by the caller; use fp8_quantize with separate
 *     workspaces for concurrent per-tensor quantizes.
 *   - A shape needing more partials than the array holds returns
 *     GS_ERR_WORKSPACE (none does: the partial count is capped at 8192).
 * Other arguments, results and errors exactly as fp8_quantize.
 */
gs_status fp8_quantize_no_workspace(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                                    fp8_format fmt, fp8_granularity g, fp8_scale_mode mode,
                                    uint8_t *codes, float *scales, int32_t *nonfinite,
                                    void *stream);

/*
 * fp8_quantize_delayed -- per-tensor FP8 quantization with delayed scaling:
 * the scale applied this step comes from a history of recent amax values,
 * so the tensor is read once.  "Why FP8 training is stable", Failure 1
 * (delayed scaling keeps a short history of recent max-abs values and
 * derives s from it; the scale applied this step reflects earlier steps), and
 * the "FP8 training" figure of "Mixed precision and FP8 training" (per
 * tensor, delayed, from recent amax).  One step:
 *   codes = cast of x with s = *scale_state (the given-scale cast of
 *           fp8_quantize: divide, clamp to +-MAX, round to nearest even);
 *   *scale_used = s (dequantize these codes with it);
 *   amax_t = largest finite |x| (0 if none);
 *   p = *history_pos mod history_len; amax_history[p] = amax_t;
 *   *history_pos = (p + 1) mod history_len;
 *   *scale_state = fl32(max(max(amax_history), fl32(1e-12)) / MAX), the
 *           scale of the next step (the maximum over the window).
 *
 *   x, x_dtype, rows, cols, fmt, codes, nonfinite: as fp8_quantize
 *              (per-tensor layout; any shape).
 *   scale_state   device FP32 [1], read and rewritten (start it at the first
 *                 step's scale, e.g. 1.0).
 *   amax_history  device FP32 [history_len], zeroed by the caller before the
 *                 first step; 1 <= history_len <= 1024.
 *   history_pos   device int32 (0 at the start).
 *   scale_used    device FP32 [1], written.
 *   workspace     >= fp8_quantize_workspace_size(rows, cols, FP8_PER_TENSOR)
 *                 bytes of device scratch (no initialisation needed).
 * Two launches on `stream` (cast + partial maxima, then the history update);
 * no host synchronisation.
 */
gs_status fp8_quantize_delayed(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                               fp8_format fmt, float *scale_state, float *amax_history,
                               int32_t history_len, int32_t *history_pos, uint8_t *codes,
                               float *scale_used, int32_t *nonfinite, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * fp8_dequantize -- out = fl32(decode(code) * s) in FP32, the canonical NaN
 * 0x7FC00000 where that is NaN ("Mixed precision and FP8 training",
 * quant(): cast back to float and multiply by the scale).  E5M2 Inf codes
 * give +-Inf * s.
 *   codes      device uint8 rows x cols (16-byte aligned); scales device
 *              FP32 in the layout of fp8_quantize (4-byte aligned); out device
 *              FP32 rows x cols (16-byte aligned).
 *   Shape rules as for fp8_quantize.
 */
gs_status fp8_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, fp8_format fmt,
                         fp8_granularity g, const float *scales, float *out, void *stream);

/*
 * fp8_dequantize_bf16 -- the same value in the BF16 compute type: fl32(
 * decode(code) * s) as fp8_dequantize computes it, then rounded to the
 * nearest BF16 value with ties to an even last bit (a value past the largest
 * BF16 becomes +-Inf); NaN is written as 0x7FC0.  The pages multiply by the
 * scale in FP32 ("Mixed precision and FP8 training", quant()); the second
 * rounding is this library's reading of handing that value to BF16 compute.
 *   codes, scales, shapes and granularities as fp8_dequantize;
 *   out        device BF16 bit patterns (uint16) rows x cols, 16-byte aligned.
 */
gs_status fp8_dequantize_bf16(const uint8_t *codes, int64_t rows, int64_t cols, fp8_format fmt,
                              fp8_granularity g, const float *scales, uint16_t *out,
                              void *stream);

/*
 * fp8_quantize_mx -- MX-style quantization: 1x32 blocks along each row, one
 * power-of-two scale per block stored as an E8M0 byte ("Mixed precision and
 * FP8 training", hardware notes: the MX formats keep one scaling factor per
 * 32 elements; the page does not define the factor's encoding).  Per block:
 *   amax = largest finite |x| (0 if none);
 *   s = the smallest power of two >= fl32(max(amax, fl32(1e-12)) / MAX)
 *       (the fp8_quantize block scale rounded up, so no finite element
 *       saturates); scales_e8m0[block] = log2(s) + 127 (the FP32 exponent
 *       field of s);
 *   codes as fp8_quantize with that s (divide, clamp, round to nearest
 *   even; NaN -> sign|0x7F).
 *   x          device BF16 or FP32 rows x cols, 16-byte aligned;
 *              cols % 32 == 0 (GS_ERR_SHAPE otherwise).
 *   codes      device uint8 rows x cols, 16-byte aligned.
 *   scales_e8m0 device uint8 [rows][cols/32].
 *   nonfinite  device int32 or NULL, set-only as in fp8_quantize.
 * One launch on `stream`.
 */
gs_status fp8_quantize_mx(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                          fp8_format fmt, uint8_t *codes, uint8_t *scales_e8m0,
                          int32_t *nonfinite, void *stream);

/*
 * fp8_dequantize_mx -- out = fl32(decode(code) * 2^(b - 127)) with b the
 * block's E8M0 byte (b = 0xFF is a NaN scale), the canonical NaN
 * 0x7FC00000 where that is NaN.  codes device uint8 rows x cols (16-byte
 * aligned, cols % 32 == 0); scales_e8m0 device uint8 [rows][cols/32]; out
 * device FP32 rows x cols (16-byte aligned).
 */
gs_status fp8_dequantize_mx(const uint8_t *codes, int64_t rows, int64_t cols, fp8_format fmt,
                            const uint8_t *scales_e8m0, float *out, void *stream);

/* Human-readable name of a status code (static string). */
const char *gs_status_string(gs_status status);

#ifdef __cplusplus
}
#endif

#endif /* GS_FP8_H */
