/*
 * synth_host.c -- seeded synthetic inputs, host side.
 *
 * Test and benchmark infrastructure: it holds none of the optimizer's
 * arithmetic.  synth_dev.hip implements the same definition on the GPU and
 * the two produce identical bits for every index, so large inputs can be made
 * in device memory while any element can be regenerated on the host.
 *
 * Definition.
 *   key(seed, stream) = mix(seed * GOLDEN + stream)
 *   h(key, i)         = mix(key + (i + 1) * GOLDEN)     (i-th splitmix64 output)
 *   mix(z)            = splitmix64 finalizer (Steele, Lea, Flood 2014)
 * Approximate normal value: the four 16-bit lanes of h are summed (an
 * Irwin-Hall sum of 4 uniforms on 0..65535, mean 131070), the centred integer
 * is converted exactly to fp32 and multiplied once by an fp32 scale
 * (sigma / 37837.2275..., the sum's standard deviation).  That single
 * multiply is the only floating-point operation.
 * bf16 values are the upper 16 bits of that fp32 value (truncation).
 * fp16 values (loss-scaled gradients): the normal value times an fp32 loss
 * scale (a second single multiply), narrowed to fp16 by truncating the
 * mantissa toward zero; magnitudes past the fp16 range become Inf and those
 * below 2^-14 are flushed to zero -- the generator's own narrowing, not the
 * round-to-nearest conversion of the method.
 * Gradient "kinds" (for the stress workload) come from a second hash stream:
 * r = (h_sel >> 32) mod 10^6 selects exact zero, a bf16 subnormal or an
 * outlier (the normal value with a larger scale) with given counts per million.
 */
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream)
{
    return mix(seed * GOLDEN + stream);
}

uint64_t synth_hash(uint64_t key, uint64_t i)
{
    return mix(key + (i + 1) * GOLDEN);
}

static inline float normal_f32(uint64_t h, float scale)
{
    int32_t s = (int32_t)(h & 0xffff) + (int32_t)((h >> 16) & 0xffff) +
                (int32_t)((h >> 32) & 0xffff) + (int32_t)(h >> 48);
    return (float)(s - 131070) * scale;
}

static inline uint16_t upper16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Grad kind thresholds, counts per million, applied in this order. */
typedef struct {
    uint32_t zero_ppm, subnormal_ppm, outlier_ppm;
} kinds;

static inline uint16_t grad_bf16(uint64_t key, uint64_t ksel, uint64_t i,
                                 float scale, float out_scale, kinds k)
{
    if (k.zero_ppm | k.subnormal_ppm | k.outlier_ppm) {
        uint64_t sel = synth_hash(ksel, i);
        uint32_t r = (uint32_t)((sel >> 32) % 1000000u);
        if (r < k.zero_ppm)
            return 0;
        r -= k.zero_ppm;
        if (r < k.subnormal_ppm)
            return (uint16_t)(((sel >> 31) & 1u) << 15 | (1u + (uint32_t)((sel >> 8) % 127u)));
        r -= k.subnormal_ppm;
        if (r < k.outlier_ppm)
            return upper16(normal_f32(synth_hash(key, i), out_scale));
    }
    return upper16(normal_f32(synth_hash(key, i), scale));
}

/* out[i] = normal value of global index base + i, i < n. */
void synth_normal_f32(float *out, int64_t n, uint64_t key, int64_t base,
                      float scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = normal_f32(synth_hash(key, (uint64_t)(base + i)), scale);
}

/* Same, at arbitrary global indices. */
void synth_normal_f32_at(float *out, const int64_t *idx, int64_t n,
                         uint64_t key, float scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = normal_f32(synth_hash(key, (uint64_t)idx[i]), scale);
}

void synth_grad_bf16(uint16_t *out, int64_t n, uint64_t key, uint64_t ksel,
                     int64_t base, float scale, float out_scale,
                     uint32_t zero_ppm, uint32_t subnormal_ppm,
                     uint32_t outlier_ppm)
{
    kinds k = {zero_ppm, subnormal_ppm, outlier_ppm};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = grad_bf16(key, ksel, (uint64_t)(base + i), scale, out_scale, k);
}

void synth_grad_bf16_at(uint16_t *out, const int64_t *idx, int64_t n,
                        uint64_t key, uint64_t ksel, float scale,
                        float out_scale, uint32_t zero_ppm,
                        uint32_t subnormal_ppm, uint32_t outlier_ppm)
{
    kinds k = {zero_ppm, subnormal_ppm, outlier_ppm};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = grad_bf16(key, ksel, (uint64_t)idx[i], scale, out_scale, k);
}

/* fp32 -> fp16 by truncation (generator only): |x| >= 65536 -> Inf, |x| < 2^-14 -> 0. */
static inline uint16_t trunc_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a >= 0x47800000u)
        return (uint16_t)(sign | 0x7c00u);
    if (a < 0x38800000u)
        return sign;
    return (uint16_t)(sign | ((a - 0x38000000u) >> 13));
}

void synth_grad_f16(uint16_t *out, int64_t n, uint64_t key, int64_t base, float scale,
                    float loss_scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = trunc_f16(normal_f32(synth_hash(key, (uint64_t)(base + i)), scale) * loss_scale);
}

void synth_grad_f16_at(uint16_t *out, const int64_t *idx, int64_t n, uint64_t key, float scale,
                       float loss_scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = trunc_f16(normal_f32(synth_hash(key, (uint64_t)idx[i]), scale) * loss_scale);
}
