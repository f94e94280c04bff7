/*
 * oracle_check.c -- the oracle (oracle/zo.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point over small seeded inputs,
 * including n = 0, M = 16, odd lengths, NaN/Inf/subnormal gradients, the fp16
 * path and the loss scaler.  Exit status 0 when nothing is reported.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void zo_bf16_to_f32_array(int64_t n, const uint16_t *in, float *out);
void zo_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out);
void zo_set_threads(int32_t n);
double zo_pow_int(double b, int64_t t);
void zo_reduce_mean_f32(int64_t n, int32_t M, const uint16_t *const *grads, float *out);
double zo_grad_sumsq(int64_t n, int32_t M, const uint16_t *const *grads);
float zo_coef_from_norm(double norm, float max_norm);
float zo_clip_coef(double sumsq, float max_norm);
int32_t zo_step_f32(int64_t n, int32_t M, const uint16_t *const *grads, float *master, float *m,
                    float *v, uint16_t *param, const uint8_t *decay, float lr, float beta1,
                    float beta2, float eps, float wd, int64_t t, int32_t use_coef, float coef);
int32_t zo_step_f64(int64_t n, int32_t M, const double *const *grads, double *master, double *m,
                    double *v, const uint8_t *decay, double lr, double beta1, double beta2,
                    double eps, double wd, int64_t t, int32_t use_coef, double coef);
void zo_f16_to_f32_array(int64_t n, const uint16_t *in, float *out);
void zo_f32_to_f16_array(int64_t n, const float *in, uint16_t *out);
float zo_inv_scale(float scale);
void zo_reduce_mean_f16(int64_t n, int32_t M, const uint16_t *const *grads, float inv_scale,
                        float *out);
double zo_grad_sumsq_f16(int64_t n, int32_t M, const uint16_t *const *grads, float inv_scale);
int32_t zo_step_f16(int64_t n, int32_t M, const uint16_t *const *grads, float *master, float *m,
                    float *v, uint16_t *param, const uint8_t *decay, float lr, float beta1,
                    float beta2, float eps, float wd, int64_t t, float inv_scale,
                    int32_t use_coef, float coef);
void zo_scaler_update(float *scale, int32_t *growth_tracker, int32_t found_inf, float growth,
                      float backoff, int32_t interval);
int32_t zo_amp_step(int64_t n, int32_t M, const uint16_t *const *grads, float *master, float *m,
                    float *v, uint16_t *param_f16, const uint8_t *decay, float lr, float beta1,
                    float beta2, float eps, float wd, float max_norm, float *scale,
                    int32_t *growth_tracker, int64_t *applied, float growth_factor,
                    float backoff_factor, int32_t growth_interval, double *norm_out);

static uint64_t rng = 0x853C49E6748FEA9Bull;
static uint32_t next_u32(void)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng >> 32);
}

int main(void)
{
    const int64_t sizes[] = {0, 1, 7, 64, 65537, 200003};
    for (int si = 0; si < 6; si++) {
        const int64_t n = sizes[si];
        for (int M = 1; M <= 16; M += 5) {
            uint16_t *g[16];
            double *gd[16];
            for (int j = 0; j < M; j++) {
                g[j] = malloc((size_t)(n ? n : 1) * 2);
                gd[j] = malloc((size_t)(n ? n : 1) * 8);
                for (int64_t i = 0; i < n; i++) {
                    uint32_t r = next_u32();
                    g[j][i] = (uint16_t)((r % 100 == 0) ? 0x7F80 : (r % 97 == 0) ? 0x0001 : (r >> 16));
                    gd[j][i] = (double)(int32_t)(r % 2001 - 1000) * 1e-6;
                }
            }
            float *p = calloc((size_t)(n ? n : 1), 4), *m = calloc((size_t)(n ? n : 1), 4);
            float *v = calloc((size_t)(n ? n : 1), 4), *avg = calloc((size_t)(n ? n : 1), 4);
            double *pd = calloc((size_t)(n ? n : 1), 8), *md = calloc((size_t)(n ? n : 1), 8);
            double *vd = calloc((size_t)(n ? n : 1), 8);
            uint16_t *b = calloc((size_t)(n ? n : 1), 2);
            uint8_t *dec = calloc((size_t)(n ? n : 1), 1);
            for (int64_t i = 0; i < n; i++) dec[i] = (uint8_t)(i & 1);
            zo_set_threads(1 + (M % 4));
            zo_reduce_mean_f32(n, M, (const uint16_t *const *)g, avg);
            const double ss = zo_grad_sumsq(n, M, (const uint16_t *const *)g);
            const float coef = zo_clip_coef(ss, 1.0f);
            for (int t = 1; t <= 3; t++) {
                if (zo_step_f32(n, M, (const uint16_t *const *)g, p, m, v, b, dec, 1e-3f, 0.9f,
                                0.95f, 1e-8f, 0.1f, t, t == 2, coef) != 0)
                    return 1;
                if (zo_step_f64(n, M, (const double *const *)gd, pd, md, vd, NULL, 1e-3, 0.9,
                                0.95, 1e-8, 0.1, t, 0, 1.0) != 0)
                    return 1;
                if (zo_step_f16(n, M, (const uint16_t *const *)g, p, m, v, b, dec, 1e-3f, 0.9f,
                                0.95f, 1e-8f, 0.1f, t, zo_inv_scale(1024.0f), 0, 1.0f) != 0)
                    return 1;
            }
            {
                float sc = 1024.0f;
                int32_t tr = 0;
                int64_t applied = 0;
                double norm = 0.0;
                for (int t = 1; t <= 3; t++)
                    if (zo_amp_step(n, M, (const uint16_t *const *)g, p, m, v, b, dec, 1e-3f,
                                    0.9f, 0.95f, 1e-8f, 0.1f, t == 2 ? 0.5f : 0.0f, &sc, &tr,
                                    &applied, 2.0f, 0.5f, 1, t == 3 ? NULL : &norm) < 0)
                        return 1;
            }
            zo_reduce_mean_f16(n, M, (const uint16_t *const *)g, zo_inv_scale(8.0f), avg);
            (void)zo_grad_sumsq_f16(n, M, (const uint16_t *const *)g, zo_inv_scale(8.0f));
            zo_bf16_to_f32_array(n, b, avg);
            zo_f32_to_bf16_array(n, avg, b);
            zo_f16_to_f32_array(n, b, avg);
            zo_f32_to_f16_array(n, avg, b);
            for (int j = 0; j < M; j++) free(g[j]), free(gd[j]);
            free(p), free(m), free(v), free(avg), free(pd), free(md), free(vd), free(b), free(dec);
        }
    }
    float scale = 65536.0f;
    int32_t tracker = 0;
    for (int i = 0; i < 1000; i++) zo_scaler_update(&scale, &tracker, (next_u32() % 7) == 0, 2.0f, 0.5f, 5);
    (void)zo_pow_int(0.999, 1000000);
    (void)zo_coef_from_norm(INFINITY, 1.0f);
    (void)zo_coef_from_norm(NAN, 1.0f);
    printf("oracle check ok\n");
    return 0;
}
