/*
 * zo.c -- the CPU oracle for the per-rank ZeRO shard step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct
 * definition the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it; the product
 * library never links, loads or calls it, and the two share no code.
 *
 * One step on one rank's flat shard of n elements computes, per element i:
 *
 *   1. g = (1/M) * sum_j grad_j[i]  -- the average of M gradient contributions
 *      (micro-batches, or data-parallel ranks for the reduce half of a
 *      reduce-scatter).  The accumulation identity is the gradient
 *      accumulation equation g = (1/M) sum_j grad l_j of Lecture04 notes,
 *      section "单卡 baseline 与 gradient accumulation 的隐藏假设"; the
 *      sum-then-divide form (add the contributions up, then divide by their
 *      count) is the DDP loop of 第7讲 CS336 并行, §6.2.  The contributions are bf16,
 *      widened exactly to fp32 and summed in fp32 in the fixed order
 *      j = 0..M-1 (fp32 reduce: 大模型基础设施工程 06, §9.1 and §15.3).
 *   2. optionally g = g * coef, coef = min(1, max_norm / (||g||_2 + 1e-6)),
 *      ||g|| over the whole (global) gradient, accumulated in fp64
 *      (gradient clipping is part of the AdamW recipe named in Lecture 9
 *      分布式训练 (CS324 notes), §7.4; the coefficient is torch's
 *      clip_grad_norm_).
 *   3. the AdamW update of zo_update.inc on the fp32 master weight and the
 *      fp32 moments m, v (16 bytes per parameter: bf16 param + bf16 grad +
 *      fp32 master, m, v -- CS324 notes §2.1; CS336 第七讲 summary, Q3).
 *   4. param = bf16(master), round to nearest even -- the buffer an
 *      all-gather would distribute after the local update (Lecture04 notes,
 *      "ZeRO-1"; CS324 notes §3.4).
 *
 * Precision.  fp32 storage and fp32 arithmetic, each operation rounded once
 * to nearest even: this file is built with -ffp-contract=off, without
 * fast-math, on SSE (no x87 excess precision), and subnormals are kept.
 * The host scalars (1-beta, bias corrections, lr/bc1, sqrt(bc2), 1-lr*wd)
 * are computed in fp64 from the fp32 hyper-parameters and rounded once to
 * fp32; beta^t is taken by fp64 binary powering (zo_pow_int).  zo_step_f64 runs the same formula entirely in fp64; it exists only
 * so the formula itself can be pinned against fp64 references.
 *
 * Thread count never changes a result: the update is elementwise, and the
 * fp64 norm is summed over fixed blocks of 65536 elements whose partial
 * sums are then added in block order.
 *
 * fp16 variant with dynamic loss scaling (the end of this file).  The pages
 * name fp16 overflow and the loss scaler that must keep up with it as the
 * hazard of 16-bit training (CS324 notes §13; 大模型基础设施工程 06, §12
 * pitfall 7) without spelling the scaler out; the reading taken is torch's
 * GradScaler: contributions of the loss scaled by `scale` are averaged in
 * fp32, multiplied by inv_scale = fp32(1/scale), and if any result is not
 * finite the step is skipped and scale *= backoff; otherwise the step runs
 * and, after growth_interval consecutive good steps, scale *= growth when
 * the grown scale is finite.  The clip, if any, uses the unscaled norm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ bf16 */

/* bf16 -> fp32: the bf16 pattern is the upper half of the fp32 pattern. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even.  NaN stays NaN (quieted). */
static uint16_t f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

void zo_bf16_to_f32_array(int64_t n, const uint16_t *in, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_to_f32(in[i]);
}

void zo_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------- threads */

void zo_set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int32_t zo_get_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------ step scalars */

typedef struct {
    float beta1, beta2, c1, c2, alpha, bhat, eps, decay_mul;
} zo_scalars_f32;

typedef struct {
    double beta1, beta2, c1, c2, alpha, bhat, eps, decay_mul;
} zo_scalars_f64;

/* b^t in fp64 by binary powering: square-and-multiply over the bits of t from
 * the lowest, each product rounded once.  A fixed sequence of IEEE multiplies,
 * so any conforming implementation gives the same bits. */
double zo_pow_int(double b, int64_t t)
{
    double r = 1.0, x = b;
    while (t > 0) {
        if (t & 1)
            r = r * x;
        x = x * x;
        t >>= 1;
    }
    return r;
}

/* fp64 evaluation of the per-step constants; t is 1-based. */
static zo_scalars_f64 scalars_f64(double lr, double beta1, double beta2,
                                  double eps, double wd, int64_t t)
{
    zo_scalars_f64 k;
    double bc1 = 1.0 - zo_pow_int(beta1, t);
    double bc2 = 1.0 - zo_pow_int(beta2, t);
    k.beta1 = beta1;
    k.beta2 = beta2;
    k.c1 = 1.0 - beta1;
    k.c2 = 1.0 - beta2;
    k.alpha = lr / bc1;
    k.bhat = sqrt(bc2);
    k.eps = eps;
    k.decay_mul = 1.0 - lr * wd;
    return k;
}

/* The same constants, each rounded once to fp32. */
static zo_scalars_f32 scalars_f32(float lr, float beta1, float beta2,
                                  float eps, float wd, int64_t t)
{
    zo_scalars_f64 d = scalars_f64(lr, beta1, beta2, eps, wd, t);
    zo_scalars_f32 k;
    k.beta1 = beta1;
    k.beta2 = beta2;
    k.c1 = (float)d.c1;
    k.c2 = (float)d.c2;
    k.alpha = (float)d.alpha;
    k.bhat = (float)d.bhat;
    k.eps = eps;
    k.decay_mul = (float)d.decay_mul;
    return k;
}

/* out = {beta1, beta2, c1, c2, alpha, bhat, eps, decay_mul} */
void zo_scalars_f32_get(float lr, float beta1, float beta2, float eps,
                        float wd, int64_t t, float *out)
{
    zo_scalars_f32 k = scalars_f32(lr, beta1, beta2, eps, wd, t);
    out[0] = k.beta1; out[1] = k.beta2; out[2] = k.c1; out[3] = k.c2;
    out[4] = k.alpha; out[5] = k.bhat; out[6] = k.eps; out[7] = k.decay_mul;
}

/* ------------------------------------------- the element update, twice */

#define ZO_REAL float
#define ZO_FN(x) x##_f32
#define ZO_SCALARS zo_scalars_f32
#define ZO_SQRT sqrtf
#include "zo_update.inc"
#undef ZO_REAL
#undef ZO_FN
#undef ZO_SCALARS
#undef ZO_SQRT

#define ZO_REAL double
#define ZO_FN(x) x##_f64
#define ZO_SCALARS zo_scalars_f64
#define ZO_SQRT sqrt
#include "zo_update.inc"
#undef ZO_REAL
#undef ZO_FN
#undef ZO_SCALARS
#undef ZO_SQRT

/* ------------------------------------------------- the M-way reduce */

/* fp32 average of M bf16 contributions, summed in order j = 0..M-1. */
static float mean_f32(const uint16_t *const *grads, int32_t M, int64_t i)
{
    float s = bf16_to_f32(grads[0][i]);
    for (int32_t j = 1; j < M; j++)
        s = s + bf16_to_f32(grads[j][i]);
    return s / (float)M;
}

void zo_reduce_mean_f32(int64_t n, int32_t M, const uint16_t *const *grads,
                        float *g_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        g_out[i] = mean_f32(grads, M, i);
}

/* ----------------------------------------------------- global norm */

#define ZO_NORM_BLOCK 65536

/* sum over i of g_i^2 in fp64, g_i the fp32 average above.  Each square of
 * an fp32 value is exact in fp64; only the additions round.  Elements are
 * summed in order inside fixed 65536-element blocks, then the block sums in
 * block order. */
double zo_grad_sumsq(int64_t n, int32_t M, const uint16_t *const *grads)
{
    if (n <= 0 || M < 1)
        return 0.0;
    int64_t nb = (n + ZO_NORM_BLOCK - 1) / ZO_NORM_BLOCK;
    double *part = (double *)malloc((size_t)nb * sizeof(double));
    if (!part)
        return NAN;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; b++) {
        int64_t lo = b * ZO_NORM_BLOCK;
        int64_t hi = lo + ZO_NORM_BLOCK < n ? lo + ZO_NORM_BLOCK : n;
        double acc = 0.0;
        for (int64_t i = lo; i < hi; i++) {
            double g = (double)mean_f32(grads, M, i);
            acc += g * g;
        }
        part[b] = acc;
    }
    double total = 0.0;
    for (int64_t b = 0; b < nb; b++)
        total += part[b];
    free(part);
    return total;
}

/* coef = min(1, max_norm / (norm + 1e-6)) in fp64, rounded once. */
float zo_coef_from_norm(double norm, float max_norm)
{
    double c = (double)max_norm / (norm + 1e-6);
    if (c > 1.0)
        c = 1.0;
    return (float)c;
}

/* the same from the sum of squares: norm = sqrt(sumsq). */
float zo_clip_coef(double sumsq, float max_norm)
{
    return zo_coef_from_norm(sqrt(sumsq), max_norm);
}

/* ------------------------------------------------------- the steps */

/*
 * One fp32 step over n elements.
 *   grads[j]  : n bf16 patterns, j < M
 *   master, m, v : fp32, updated in place
 *   param     : n bf16 patterns written (may be NULL)
 *   decay     : per-element flag (nonzero: weight decay applies); NULL = all
 *   use_coef  : nonzero multiplies g by coef after averaging
 * Returns 0, or -1 for bad arguments.
 */
int32_t zo_step_f32(int64_t n, int32_t M, const uint16_t *const *grads,
                    float *master, float *m, float *v, uint16_t *param,
                    const uint8_t *decay, float lr, float beta1, float beta2,
                    float eps, float wd, int64_t t, int32_t use_coef,
                    float coef)
{
    if (n < 0 || M < 1 || t < 1 || !grads || !master || !m || !v)
        return -1;
    zo_scalars_f32 k = scalars_f32(lr, beta1, beta2, eps, wd, t);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float g = mean_f32(grads, M, i);
        if (use_coef)
            g = g * coef;
        float d = (decay == NULL || decay[i]) ? k.decay_mul : 1.0f;
        update_f32(g, &master[i], &m[i], &v[i], &k, d);
        if (param)
            param[i] = f32_to_bf16(master[i]);
    }
    return 0;
}

/* The same step entirely in fp64, on fp64 gradient contributions. */
int32_t zo_step_f64(int64_t n, int32_t M, const double *const *grads,
                    double *master, double *m, double *v,
                    const uint8_t *decay, double lr, double beta1,
                    double beta2, double eps, double wd, int64_t t,
                    int32_t use_coef, double coef)
{
    if (n < 0 || M < 1 || t < 1 || !grads || !master || !m || !v)
        return -1;
    zo_scalars_f64 k = scalars_f64(lr, beta1, beta2, eps, wd, t);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double s = grads[0][i];
        for (int32_t j = 1; j < M; j++)
            s = s + grads[j][i];
        double g = s / (double)M;
        if (use_coef)
            g = g * coef;
        double d = (decay == NULL || decay[i]) ? k.decay_mul : 1.0;
        update_f64(g, &master[i], &m[i], &v[i], &k, d);
    }
    return 0;
}

/* --------------------------------- fp16 variant with dynamic loss scaling */

/* fp16 -> fp32 (exact). */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, mant = h & 0x3ffu;
    uint32_t u;
    if (e == 0x1f) {
        u = sign | 0x7f800000u | (mant << 13);             /* Inf / NaN */
    } else if (e != 0) {
        u = sign | ((e + 112u) << 23) | (mant << 13);      /* normal: rebias 15 -> 127 */
    } else if (mant == 0) {
        u = sign;                                         /* +-0 */
    } else {                                              /* subnormal: mant * 2^-24 */
        float f = (float)mant * 5.9604644775390625e-8f;    /* exact: mant < 2^10 */
        memcpy(&u, &f, sizeof u);
        u |= sign;
    }
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> fp16, round to nearest, ties to even; overflow to Inf; NaN stays
 * a quiet NaN with the top payload bits. */
static uint16_t f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u)                                  /* NaN */
        return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x1ffu));
    if (a >= 0x477ff000u)                                 /* >= 65520: rounds to Inf */
        return (uint16_t)(sign | 0x7c00u);
    if (a >= 0x38800000u) {                               /* fp16 normal range */
        uint32_t m = a - 0x38000000u;                     /* rebias 127 -> 15 */
        uint32_t r = (m + 0xfffu + ((m >> 13) & 1u)) >> 13;
        return (uint16_t)(sign | r);
    }
    if (a <= 0x33000000u)                                 /* <= 2^-25: rounds to 0 */
        return sign;
    {                                                     /* fp16 subnormal */
        uint32_t e = a >> 23, mant = (a & 0x7fffffu) | 0x800000u;
        uint32_t sh = 126u - e;                           /* value / 2^-24 = mant >> sh */
        uint32_t q = mant >> sh, rem = mant & ((1u << sh) - 1u), half = 1u << (sh - 1u);
        if (rem > half || (rem == half && (q & 1u)))
            q++;
        return (uint16_t)(sign | q);
    }
}

void zo_f16_to_f32_array(int64_t n, const uint16_t *in, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = f16_to_f32(in[i]);
}

void zo_f32_to_f16_array(int64_t n, const float *in, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f32_to_f16(in[i]);
}

/* inv_scale = fp32(1 / scale), the reciprocal taken in fp64. */
float zo_inv_scale(float scale)
{
    return (float)(1.0 / (double)scale);
}

/* The unscaled fp32 average of M fp16 contributions: ((sum_j g_j) / M) * inv_scale. */
static float mean_f16_unscaled(const uint16_t *const *grads, int32_t M, int64_t i,
                               float inv_scale)
{
    float s = f16_to_f32(grads[0][i]);
    for (int32_t j = 1; j < M; j++)
        s = s + f16_to_f32(grads[j][i]);
    float g = s / (float)M;
    return g * inv_scale;
}

void zo_reduce_mean_f16(int64_t n, int32_t M, const uint16_t *const *grads, float inv_scale,
                        float *g_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        g_out[i] = mean_f16_unscaled(grads, M, i, inv_scale);
}

/* Sum of squares of the unscaled average (fp64, fixed blocks as above); it is
 * not finite exactly when some unscaled element is not finite (the found-inf
 * test). */
double zo_grad_sumsq_f16(int64_t n, int32_t M, const uint16_t *const *grads, float inv_scale)
{
    if (n <= 0 || M < 1)
        return 0.0;
    int64_t nb = (n + ZO_NORM_BLOCK - 1) / ZO_NORM_BLOCK;
    double *part = (double *)malloc((size_t)nb * sizeof(double));
    if (!part)
        return NAN;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; b++) {
        int64_t lo = b * ZO_NORM_BLOCK;
        int64_t hi = lo + ZO_NORM_BLOCK < n ? lo + ZO_NORM_BLOCK : n;
        double acc = 0.0;
        for (int64_t i = lo; i < hi; i++) {
            double g = (double)mean_f16_unscaled(grads, M, i, inv_scale);
            acc += g * g;
        }
        part[b] = acc;
    }
    double total = 0.0;
    for (int64_t b = 0; b < nb; b++)
        total += part[b];
    free(part);
    return total;
}

/* One fp32 step on fp16 contributions of a loss scaled by 1/inv_scale; the
 * param copy is fp16.  The caller skips the call when found-inf holds. */
int32_t zo_step_f16(int64_t n, int32_t M, const uint16_t *const *grads, float *master, float *m,
                    float *v, uint16_t *param_f16, const uint8_t *decay, float lr, float beta1,
                    float beta2, float eps, float wd, int64_t t, float inv_scale,
                    int32_t use_coef, float coef)
{
    if (n < 0 || M < 1 || t < 1 || !grads || !master || !m || !v)
        return -1;
    zo_scalars_f32 k = scalars_f32(lr, beta1, beta2, eps, wd, t);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float g = mean_f16_unscaled(grads, M, i, inv_scale);
        if (use_coef)
            g = g * coef;
        float d = (decay == NULL || decay[i]) ? k.decay_mul : 1.0f;
        update_f32(g, &master[i], &m[i], &v[i], &k, d);
        if (param_f16)
            param_f16[i] = f32_to_f16(master[i]);
    }
    return 0;
}

/* The loss-scale update after a step: found_inf -> scale *= backoff and the
 * growth count restarts; otherwise the count grows and, on reaching
 * growth_interval, the count restarts and scale *= growth -- unless the grown
 * scale would not be finite, in which case the scale stays (torch's
 * GradScaler: a scale that overflowed to Inf would zero every later unscaled
 * gradient). */
void zo_scaler_update(float *scale, int32_t *growth_tracker, int32_t found_inf,
                      float growth_factor, float backoff_factor, int32_t growth_interval)
{
    if (found_inf) {
        *scale = *scale * backoff_factor;
        *growth_tracker = 0;
    } else {
        int32_t good = *growth_tracker + 1;
        if (good == growth_interval) {
            float grown = *scale * growth_factor;
            if (isfinite(grown))
                *scale = grown;
            *growth_tracker = 0;
        } else {
            *growth_tracker = good;
        }
    }
}

/* One whole loss-scaled step, in the order torch's GradScaler drives an
 * optimizer: unscale (inv_scale = fp32(1/scale)), found-inf = the fp64 sum of
 * squares of the unscaled average is not finite, the optional clip on the
 * unscaled norm, the update at t = applied + 1 unless found-inf (a skipped
 * step does not advance t), then the scale update.  *norm_out (optional)
 * receives sqrt of that sum of squares.  Returns 1 when the step was skipped,
 * 0 when applied, -1 for bad arguments. */
int32_t zo_amp_step(int64_t n, int32_t M, const uint16_t *const *grads, float *master, float *m,
                    float *v, uint16_t *param_f16, const uint8_t *decay, float lr, float beta1,
                    float beta2, float eps, float wd, float max_norm, float *scale,
                    int32_t *growth_tracker, int64_t *applied, float growth_factor,
                    float backoff_factor, int32_t growth_interval, double *norm_out)
{
    if (n < 0 || M < 1 || !grads || !master || !m || !v || !scale || !growth_tracker ||
        !applied)
        return -1;
    float inv = zo_inv_scale(*scale);
    double sumsq = zo_grad_sumsq_f16(n, M, grads, inv);
    int32_t found_inf = !isfinite(sumsq);
    double norm = sqrt(sumsq);
    if (norm_out)
        *norm_out = norm;
    if (!found_inf) {
        int32_t use_coef = max_norm > 0.0f;
        float coef = use_coef ? zo_coef_from_norm(norm, max_norm) : 1.0f;
        if (zo_step_f16(n, M, grads, master, m, v, param_f16, decay, lr, beta1, beta2, eps, wd,
                        *applied + 1, inv, use_coef, coef) != 0)
            return -1;
        *applied += 1;
    }
    zo_scaler_update(scale, growth_tracker, found_inf, growth_factor, backoff_factor,
                     growth_interval);
    return found_inf;
}
