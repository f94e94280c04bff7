/*
 * abi_check.c -- the C ABI used from plain C with the HIP runtime alone (no
 * Python, no torch): one hipMalloc'ed slab placed by zs_slab_layout, a plan, a
 * context, three steps (the second clipped), checked bit for bit against the CPU oracle
 * (oracle/libzo.so, test infrastructure) on the same inputs.  Then the
 * allocation-free step (zero_shard_step_static) continues the same state: a
 * first call made under capture is refused, then it runs once
 * eagerly, then two steps (one clipped) captured into a HIP graph and replayed
 * twice, with an eager context step between the replays; every replay is
 * checked bit for bit against the oracle.  Exit status 0 on agreement.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/zeroshard.h"

/* the oracle entry points this check uses (oracle/zo.c) */
int32_t zo_step_f32(int64_t n, int32_t M, const uint16_t *const *grads, float *master, float *m,
                    float *v, uint16_t *param, const uint8_t *decay, float lr, float beta1,
                    float beta2, float eps, float wd, int64_t t, int32_t use_coef, float coef);
double zo_grad_sumsq(int64_t n, int32_t M, const uint16_t *const *grads);
float zo_coef_from_norm(double norm, float max_norm);

#define M 3
#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            return 2;                                                                 \
        }                                                                             \
    } while (0)
#define CHECK_ZS(x)                                                                  \
    do {                                                                             \
        int r_ = (x);                                                                \
        if (r_ < 0) {                                                                \
            fprintf(stderr, "%s:%d: %s (%d)\n", __FILE__, __LINE__,                  \
                    zero_shard_last_error(), r_);                                    \
            return 2;                                                                \
        }                                                                            \
    } while (0)

/* input values only: a 64-bit LCG (Knuth's MMIX constants) */
static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static float uniform_pm1(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((int32_t)(lcg >> 32)) * (1.0f / 2147483648.0f);
}
static uint16_t bf16_trunc(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

/* device state against the oracle's host state, bit for bit */
static int same_as_oracle(const char *what, int64_t S, hipStream_t stream, const float *d_master,
                          const float *d_m, const float *d_v, const void *d_param,
                          const float *master, const float *m, const float *v,
                          const uint16_t *param, float *got_master, float *got_m, float *got_v,
                          uint16_t *got_param)
{
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(got_master, d_master, S * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(got_m, d_m, S * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(got_v, d_v, S * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(got_param, d_param, S * 2, hipMemcpyDeviceToHost));
    if (memcmp(got_master, master, S * 4) || memcmp(got_m, m, S * 4) ||
        memcmp(got_v, v, S * 4) || memcmp(got_param, param, S * 2)) {
        fprintf(stderr, "%s: device state differs from the oracle\n", what);
        return 1;
    }
    return 0;
}

int main(void)
{
    const int64_t numel[] = {1000, 1, 64, 70001, 5, 4096, 333};
    const uint8_t decay[] = {1, 0, 1, 0, 1, 1, 0};
    const int64_t n_tensors = 7;
    zs_plan *plan = NULL;
    CHECK_ZS(zs_plan_create(numel, decay, n_tensors, 3, 1, 25000000, 64, &plan));
    int64_t S, n_seg, n_runs, padded, n_buckets;
    CHECK_ZS(zs_plan_query(plan, &S, &n_seg, &n_runs, &padded, &n_buckets));

    /* host inputs: masters and contributions, zero on padding; the decay mask */
    float *master = calloc(S, 4), *m = calloc(S, 4), *v = calloc(S, 4);
    float *got_master = malloc(S * 4), *got_m = malloc(S * 4), *got_v = malloc(S * 4);
    uint16_t *param = calloc(S, 2), *got_param = malloc(S * 2);
    uint8_t *mask = calloc(S, 1);
    uint16_t *grads[M];
    for (int j = 0; j < M; j++) grads[j] = calloc(S, 2);
    if (!master || !m || !v || !got_master || !got_m || !got_v || !param || !got_param || !mask)
        return 2;
    for (int64_t s = 0; s < n_seg; s++) {
        int64_t off, len, tensor, toff;
        int32_t dec;
        CHECK_ZS(zs_plan_segment(plan, s, &off, &len, &tensor, &toff, &dec));
        for (int64_t i = off; i < off + len; i++) {
            mask[i] = (uint8_t)dec;
            if (tensor < 0) continue; /* padding stays zero */
            master[i] = 0.02f * uniform_pm1();
            for (int j = 0; j < M; j++) grads[j][i] = bf16_trunc(1e-3f * uniform_pm1());
        }
    }

    /* device buffers: one slab, owned here, started on a 2 MiB boundary */
    void *d_param, *d_ws, *d_grads[M];
    float *d_master, *d_m, *d_v;
    const size_t ws_bytes = zs_workspace_bytes(plan, M, 0);
    size_t offs[5 + M], slab_bytes = 0;
    CHECK_ZS(zs_slab_layout(plan, M, 0, M, offs, &slab_bytes));
    const size_t period = (size_t)1 << 21;
    char *slab = NULL;
    CHECK_HIP(hipMalloc((void **)&slab, slab_bytes + period));
    char *base = slab + ((period - (uintptr_t)slab % period) % period);
    d_param = base + offs[0];
    d_master = (float *)(base + offs[1]);
    d_m = (float *)(base + offs[2]);
    d_v = (float *)(base + offs[3]);
    for (int j = 0; j < M; j++) {
        d_grads[j] = base + offs[4 + j];
        CHECK_HIP(hipMemcpy(d_grads[j], grads[j], S * 2, hipMemcpyHostToDevice));
    }
    d_ws = base + offs[4 + M];
    CHECK_HIP(hipMemcpy(d_master, master, S * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_m, 0, S * 4));
    CHECK_HIP(hipMemset(d_v, 0, S * 4));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    zs_ctx *ctx = NULL;
    CHECK_ZS(zero_shard_init(&ctx, plan, M, d_param, d_master, d_m, d_v, d_ws, ws_bytes, stream,
                             0));

    /* a rejected call leaves a message and enqueues nothing */
    if (zero_shard_step(ctx, (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 0,
                        0.0f, NULL) != ZS_EINVAL ||
        !zero_shard_last_error()[0]) {
        fprintf(stderr, "step 0 was not rejected\n");
        return 1;
    }

    const uint16_t *const *gp = (const uint16_t *const *)grads;
    for (int t = 1; t <= 3; t++) {
        const float max_norm = (t == 2) ? 0.05f : 0.0f;
        double norm = -1.0;
        CHECK_ZS(zero_shard_step(ctx, (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f, 1e-8f,
                                 0.1f, t, max_norm, &norm));
        const double want = sqrt(zo_grad_sumsq(S, M, gp));
        if (fabs(norm - want) > 1e-12 * want) {
            fprintf(stderr, "step %d: norm %.17g, oracle %.17g\n", t, norm, want);
            return 1;
        }
        const int use_coef = max_norm > 0.0f;
        const float coef = use_coef ? zo_coef_from_norm(norm, max_norm) : 1.0f;
        if (zo_step_f32(S, M, gp, master, m, v, param, mask, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, t,
                        use_coef, coef) != 0)
            return 2;
        char what[32];
        snprintf(what, sizeof what, "step %d", t);
        if (same_as_oracle(what, S, stream, d_master, d_m, d_v, d_param, master, m, v, param,
                           got_master, got_m, got_v, got_param))
            return 1;
    }

    /* the allocation-free step on the same state: its first call on the device runs
       eagerly (it resolves the static scratch there), the next two are captured */
    const double norm_oracle = sqrt(zo_grad_sumsq(S, M, gp));
    const float coef_oracle = zo_coef_from_norm(norm_oracle, 0.05f);
    {
        /* made while the stream captures, that first call is refused and leaves the
           capture intact */
        hipGraph_t empty = NULL;
        CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
        const int rc = zero_shard_step_static(plan, M, d_param, d_master, d_m, d_v,
                                              (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f,
                                              1e-8f, 0.1f, 4, 0.0f, stream);
        CHECK_HIP(hipStreamEndCapture(stream, &empty));
        CHECK_HIP(hipGraphDestroy(empty));
        if (rc != ZS_EINVAL || !strstr(zero_shard_last_error(), "outside graph capture")) {
            fprintf(stderr, "first static call under capture returned %d: %s\n", rc,
                    zero_shard_last_error());
            return 1;
        }
    }
    CHECK_ZS(zero_shard_step_static(plan, M, d_param, d_master, d_m, d_v,
                                    (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f,
                                    4, 0.0f, stream));
    if (zo_step_f32(S, M, gp, master, m, v, param, mask, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 4, 0,
                    1.0f) != 0)
        return 2;
    if (same_as_oracle("static step 4", S, stream, d_master, d_m, d_v, d_param, master, m, v,
                       param, got_master, got_m, got_v, got_param))
        return 1;
    hipGraph_t graph = NULL;
    hipGraphExec_t exec = NULL;
    CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
    int rc5 = zero_shard_step_static(plan, M, d_param, d_master, d_m, d_v,
                                     (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f, 1e-8f,
                                     0.1f, 5, 0.05f, stream);
    int rc6 = zero_shard_step_static(plan, M, d_param, d_master, d_m, d_v,
                                     (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f, 1e-8f,
                                     0.1f, 6, 0.0f, stream);
    CHECK_HIP(hipStreamEndCapture(stream, &graph));
    CHECK_ZS(rc5);
    CHECK_ZS(rc6);
    CHECK_HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
    for (int replay = 1; replay <= 2; replay++) {
        CHECK_HIP(hipGraphLaunch(exec, stream));
        if (zo_step_f32(S, M, gp, master, m, v, param, mask, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 5,
                        1, coef_oracle) != 0 ||
            zo_step_f32(S, M, gp, master, m, v, param, mask, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 6,
                        0, 1.0f) != 0)
            return 2;
        char what[48];
        snprintf(what, sizeof what, "graph replay %d (static steps 5, 6)", replay);
        if (same_as_oracle(what, S, stream, d_master, d_m, d_v, d_param, master, m, v, param,
                           got_master, got_m, got_v, got_param))
            return 1;
        if (replay == 1) {
            /* eager work of the program's own between the replays */
            CHECK_ZS(zero_shard_step(ctx, (const void *const *)d_grads, 1e-3f, 0.9f, 0.95f,
                                     1e-8f, 0.1f, 7, 0.0f, NULL));
            if (zo_step_f32(S, M, gp, master, m, v, param, mask, 1e-3f, 0.9f, 0.95f, 1e-8f,
                            0.1f, 7, 0, 1.0f) != 0)
                return 2;
            if (same_as_oracle("context step 7", S, stream, d_master, d_m, d_v, d_param, master,
                               m, v, param, got_master, got_m, got_v, got_param))
                return 1;
        }
    }
    CHECK_HIP(hipGraphExecDestroy(exec));
    CHECK_HIP(hipGraphDestroy(graph));
    const void *pp = NULL;
    int64_t plen = 0;
    CHECK_ZS(zero_shard_params(ctx, &pp, &plen));
    if (pp != d_param || plen != S) {
        fprintf(stderr, "zero_shard_params disagrees\n");
        return 1;
    }
    zero_shard_destroy(ctx);
    zs_plan_destroy(plan);
    CHECK_HIP(hipStreamDestroy(stream));
    for (int j = 0; j < M; j++) free(grads[j]);
    CHECK_HIP(hipFree(slab));
    free(master), free(m), free(v), free(got_master), free(got_m), free(got_v);
    free(param), free(got_param), free(mask);
    printf("c-abi check ok: S=%lld, M=%d, 3 context steps (one clipped), the allocation-free "
           "step eagerly and from a HIP graph replayed twice, bit-identical to the oracle\n",
           (long long)S, M);
    return 0;
}
