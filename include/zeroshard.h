/*
 * zeroshard.h -- C ABI of the fused per-rank ZeRO shard step for MI355X (gfx950).
 *
 * What the library computes.  One data-parallel rank owns 1/N of the flat
 * parameter space.  Per optimizer step it
 *   (a) reduces M bf16 gradient contributions of its shard into their fp32
 *       average g = (1/M) sum_j grad_j, summed in the fixed order j = 0..M-1
 *       -- the gradient-accumulation identity (Lecture04 notes, section
 *       "单卡 baseline 与 gradient accumulation 的隐藏假设", equation for g)
 *       and the reduce half of a reduce-scatter, after which each rank holds
 *       the reduced gradient of exactly the slice it owns (Lecture04 notes,
 *       "ZeRO-1"; CS324 notes §3.4; CS336 第七讲 summary, Q2);
 *   (b) optionally scales g by min(1, max_norm / (||g|| + 1e-6)), the norm
 *       accumulated in fp64 (gradient clipping of the AdamW recipe, CS324
 *       notes §7.4);
 *   (c) applies AdamW to the fp32 master weight and fp32 moments m, v of its
 *       shard -- m and v follow the Adam formula, only their ownership is
 *       sharded (Lecture04 notes, "ZeRO-1"), under the 16-bytes-per-parameter
 *       layout bf16 param + bf16 grad + fp32 master, m, v (CS324 notes §2.1;
 *       CS336 第七讲 summary, Q3);
 *   (d) writes the bf16 re-cast of the new master (round to nearest even),
 *       the buffer the all-gather then distributes (Lecture04 notes, "ZeRO-1").
 * Per element, every operation is one IEEE fp32 operation rounded to nearest:
 *   g   = (sum_j grad_j) / M            [* coef]
 *   m'  = beta1*m + (1-beta1)*g
 *   v'  = beta2*v + (1-beta2)*(g*g)
 *   den = sqrt(v') / sqrt(1-beta2^t) + eps
 *   p'  = p*(1 - lr*wd) - (lr/(1-beta1^t)) * (m'/den)
 *   param = bf16_rne(p')
 * with the per-step constants computed in fp64 on the host and rounded once
 * to fp32.  Division and square root are correctly rounded; nothing is
 * contracted into FMAs; subnormals are kept.
 *
 * Layout.  A plan flattens an ordered tensor list into buckets (tensors at
 * multiples of `align` elements, a bucket closed when the next tensor would
 * pass `bucket_cap` elements, a larger tensor alone), pads every bucket to a
 * multiple of world_size*align, and gives rank r slice r of every bucket
 * (大模型基础设施工程 06, §6.1 gradient buckets and §11.3 contiguous
 * gradients; cutting flat buffers is legal because AdamW is elementwise,
 * CS324 notes §3.4).  Every per-element array of the rank -- param, master,
 * m, v and each grads[j] -- is one flat array of shard_len elements in that
 * same order.  Padding elements must be zero in every array; the step keeps
 * them zero.
 *
 * Conventions.
 *   - Pointers named *_dev or taking buffers are device pointers; the caller
 *     allocates and owns every device buffer (grads, param, master, moments,
 *     workspace).  The library allocates or frees device memory only in the
 *     optional zs_device_alloc_contiguous / zs_device_free.
 *     zs_plan and zs_ctx are host objects owned by the library, released by
 *     their destroy calls.
 *   - Device buffers must be 16-byte aligned; the workspace 256-byte aligned.
 *   - `stream` is a hipStream_t handle (NULL: the null stream).  Calls
 *     enqueue work and return without waiting, except where stated.
 *   - Return value: 0 = ZS_OK; positive = warning; negative = error, with a
 *     message in zero_shard_last_error().  ZS_EINVAL, ZS_ENOMEM and ZS_ESTATE
 *     are found before anything is enqueued (state unchanged).  ZS_EHIP from
 *     a later kernel launch of a call can leave that call's earlier kernels
 *     enqueued; a HIP launch error usually means the device is unusable.
 *   - A context is used by one host thread at a time.
 */
#ifndef ZEROSHARD_H
#define ZEROSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zs_plan zs_plan; /* host-side layout plan */
typedef struct zs_ctx zs_ctx;   /* one rank's shard state bound to device buffers */

enum {
    ZS_OK = 0,
    ZS_NONFINITE = 1,  /* warning: the gradient norm is NaN or Inf */
    ZS_EINVAL = -1,    /* invalid argument */
    ZS_ENOMEM = -2,    /* host allocation failed */
    ZS_EHIP = -3,      /* a HIP runtime call failed */
    ZS_ESTATE = -4     /* object in the wrong state for the call */
};

/* zero_shard_init flags */
#define ZS_SKIP_NONFINITE 1u /* non-finite norm: the step leaves every array untouched */
#define ZS_FP16 2u           /* gradients and the param copy are fp16 (zero_shard_step_amp) */
/* When a call runs the norm pass (clip, grad_norm_out or ZS_SKIP_NONFINITE in
 * zero_shard_step; always in zero_shard_step_amp), that pass also stores each
 * element's averaged gradient (fp32, unscaled) in the workspace, and the step
 * reads those 4 bytes instead of the M contributions again.  Gradient bytes per
 * element go from 2M + 2M to 2M + 4 + 4: fewer for M > 4.  The workspace grows
 * by 4 * shard_len bytes.  Results are bit-identical either way. */
#define ZS_STAGE_AVERAGE 4u

/* Device state of the dynamic loss scaler (16 bytes of caller-owned device
 * memory, 16-byte aligned), read and updated by zero_shard_step_amp. */
typedef struct zs_amp_state {
    float scale;            /* the loss scale the next gradients carry */
    int32_t growth_tracker; /* consecutive steps without Inf/NaN */
    int64_t applied_steps;  /* optimizer steps applied (skipped ones do not count) */
} zs_amp_state;

#define ZS_MAX_M 16

/* ------------------------------------------------------------------ plan */

/*
 * Builds the layout of rank `rank` of `world_size` for tensors numel[0..n_tensors)
 * (element counts, forward order; 0 allowed) with weight-decay flags decay[]
 * (nonzero: decayed).  The layout is the flat gradient buckets of
 * 大模型基础设施工程 06, §6.1 (buckets closed at a size cap, in forward
 * order), kept as contiguous flat buffers (§11.3, contiguous_gradients), each
 * bucket cut into world_size equal slices of which this rank owns slice
 * `rank` -- the ZeRO partition of CS324 notes §3.4, where cutting flat buffers
 * is legal because AdamW acts element by element.  bucket_cap >= 1 elements; align a multiple of 8 (64 in
 * the reference workloads: 128 B of bf16, 256 B of fp32).
 * On success *out owns a new plan.  Errors: ZS_EINVAL (bad sizes, flags array
 * missing, geometry), ZS_ENOMEM.
 */
int zs_plan_create(const int64_t *numel, const uint8_t *decay, int64_t n_tensors,
                   int32_t world_size, int32_t rank, int64_t bucket_cap, int32_t align,
                   zs_plan **out);

/* Sizes of the plan (the partition of 大模型基础设施工程 06, §6.1 and §11.3, and
 * CS324 notes §3.4, as built by zs_plan_create).  Any output pointer may be NULL.
 *   shard_len    elements of this rank's flat shard (a multiple of align)
 *   n_segments   maximal runs of one tensor, or of padding, in the shard
 *   n_runs       maximal stretches of one weight-decay flag (padding joins a
 *                neighbour); the step kernel looks each tile's flag up here
 *   padded_total elements of all buckets together (shard_len * world_size)
 *   n_buckets    number of buckets */
int zs_plan_query(const zs_plan *plan, int64_t *shard_len, int64_t *n_segments,
                  int64_t *n_runs, int64_t *padded_total, int64_t *n_buckets);

/* Where tensor `tensor` lies in this rank's shard: elements
 * [tensor_off, tensor_off + len) of the tensor sit at [shard_off, shard_off + len).
 * len = 0 when this rank owns none of it. */
int zs_plan_tensor_slice(const zs_plan *plan, int64_t tensor, int64_t *shard_off,
                         int64_t *tensor_off, int64_t *len);

/* Segment i in shard order.  tensor = -1 for padding (tensor_off 0, decay 0). */
int zs_plan_segment(const zs_plan *plan, int64_t i, int64_t *shard_off, int64_t *len,
                    int64_t *tensor, int64_t *tensor_off, int32_t *decay);

/* Bucket b: its start in the flat (all-ranks) order and its padded length. */
int zs_plan_bucket(const zs_plan *plan, int64_t b, int64_t *flat_off, int64_t *len);

/* Weight-decay run i: shard offset, length, flag.  Runs partition the shard. */
int zs_plan_run(const zs_plan *plan, int64_t i, int64_t *shard_off, int64_t *len,
                int32_t *decay);

/* Resident model-state bytes of this rank at ZeRO stage 0..3 under 16 B/param
 * (CS324 notes §2.1, exercise 1; Lecture04 notes, ZeRO-1/ZeRO-2 formulas):
 * stage 0: 16*Psi; 1: 4*Psi + 12*S; 2: 2*Psi + 14*S; 3: 16*S,
 * Psi = sum of numel, S = shard_len. */
int zs_plan_state_bytes(const zs_plan *plan, int32_t stage, int64_t *bytes);

void zs_plan_destroy(zs_plan *plan);

/* Device workspace a context of this plan needs with these init flags (run
 * table, piece table, norm partials, clip scalars and, with ZS_STAGE_AVERAGE,
 * 4 * shard_len bytes of staged averages), in bytes; 0 if plan is NULL.  M is
 * accepted for forward compatibility and does not change the size. */
size_t zs_workspace_bytes(const zs_plan *plan, int32_t M, uint32_t flags);

/*
 * Placement of one rank's arrays in a single device allocation (the 16-byte-
 * per-parameter state of CS324 notes §2.1 plus the M gradient contributions,
 * kept in flat contiguous buffers as with contiguous_gradients in
 * 大模型基础设施工程 06, §11.3).
 *
 * A step streams every one of these arrays at the same element index.  When
 * all of them start on 2 MiB boundaries, as separate large allocations do, the
 * step on MI355X measured 0.2% to 6% slower (shard sizes 164M to 6.7G
 * elements) than with starts staggered by distinct multiples of 4 KiB.  This
 * helper computes such a staggered placement; using it is optional.
 *
 * Fills offsets[0 .. 4 + n_grads], byte offsets from the start of the slab:
 *   [0] param (shard_len 16-bit elements), [1] master, [2] exp_avg,
 *   [3] exp_avg_sq (shard_len floats each), [4 .. 3 + n_grads] gradient
 *   contribution buffers (shard_len 16-bit elements each), [4 + n_grads] the
 *   workspace (zs_workspace_bytes(plan, M, flags) bytes),
 * and *slab_bytes with the size of the slab.  Array i starts 4 KiB * i past a
 * 2 MiB boundary of the slab, so the slab itself should start on a 2 MiB
 * boundary (any 256-byte aligned start is still correct, only the stagger is
 * lost).  n_grads in [0, M]: contributions placed elsewhere are left out.  The
 * caller allocates and owns the slab.  Errors: ZS_EINVAL (offsets and
 * *slab_bytes untouched).
 */
int zs_slab_layout(const zs_plan *plan, int32_t M, uint32_t flags, int32_t n_grads,
                   size_t *offsets, size_t *slab_bytes);

/* ------------------------------------------------------------ the step */

/*
 * The pages define no interface for creating or releasing this state (they
 * describe the per-rank update, not an API); these two calls are this
 * library's own.
 *
 * Binds a context to one rank's device buffers (each shard_len elements):
 * param_bf16 (bf16, written by every step), master, exp_avg, exp_avg_sq
 * (fp32, read and written), and a workspace of zs_workspace_bytes(plan, M, flags)
 * bytes, 256-byte aligned.
 * The caller initialises master, sets exp_avg = exp_avg_sq = 0 and zeroes
 * the padding; param_bf16 is output only.  M in [1, ZS_MAX_M] is the number of
 * gradient contributions each step reduces.  flags: any of ZS_SKIP_NONFINITE,
 * ZS_FP16, ZS_STAGE_AVERAGE (0 for none).
 * Uploads the run table on `stream` and waits for that copy.  The plan may
 * be destroyed afterwards.  Errors: ZS_EINVAL, ZS_ENOMEM, ZS_EHIP.
 *
 * The streaming kernels cap their resident workgroups per CU through an LDS
 * reservation they never use.  Every reservation the context will launch
 * with, plus the kernels' static LDS, is checked here against the current
 * device's per-workgroup LDS limit (queried); ZS_EINVAL if one does not fit,
 * so no launch ever asks for more.
 *
 * Read from the environment at this call (zero_offload_init reads both too):
 *   ZS_WAVES_PER_CU           resident waves per CU of the step kernels, 3..64,
 *                             or 0 for no cap; unset: a measured table by M and
 *                             shard size.  Any other value is ZS_EINVAL.
 *   ZS_MAX_GROUPS_PER_LAUNCH  work-groups per kernel launch, > 0.  A grid larger
 *                             than one dispatch carries (2^32 - 1 work-items,
 *                             reached by shards beyond 2^34 elements) is always
 *                             issued as consecutive launches; this lowers the
 *                             slice size, which lets tests split small shards.
 *                             Results do not depend on it.
 */
int zero_shard_init(zs_ctx **out, const zs_plan *plan, int32_t M, void *param_bf16,
                    float *master, float *exp_avg, float *exp_avg_sq, void *workspace,
                    size_t workspace_bytes, void *stream, uint32_t flags);

/*
 * Enqueues one optimizer step.  grads: host array of M device pointers, each
 * to shard_len bf16 values (this rank's slice of contribution j).
 * Hyper-parameters: lr >= 0, beta1 and beta2 in [0, 1), eps > 0,
 * weight_decay >= 0, all finite; step >= 1 is the 1-based step number.
 * max_grad_norm > 0 enables the global-norm clip of this shard (for N > 1 the
 * caller uses zero_shard_grad_sumsq + zero_shard_step_global_norm instead);
 * <= 0 disables it.  grad_norm_out: optional host pointer; when non-NULL the
 * call waits for the stream and stores ||g||_2 of this shard (fp64).
 * Returns ZS_OK, ZS_NONFINITE (only when grad_norm_out is given and the norm
 * is not finite), or an error.  With ZS_SKIP_NONFINITE and a norm computed
 * (clip on, or grad_norm_out given), a non-finite norm turns the update into
 * a no-op on the device; otherwise NaN/Inf propagate as in torch.
 */
int zero_shard_step(zs_ctx *ctx, const void *const *grads, float lr, float beta1, float beta2,
                    float eps, float weight_decay, int64_t step, float max_grad_norm,
                    double *grad_norm_out);

/*
 * Multi-rank clip, part 1: enqueues sum_i g_i^2 (fp64) of this shard into the
 * device double *sumsq_dev (g as in the step, before clipping).  The caller
 * sums these partials over ranks (a scalar all-reduce) and passes the global
 * value to part 2.  Errors: ZS_EINVAL, ZS_EHIP.
 */
int zero_shard_grad_sumsq(zs_ctx *ctx, const void *const *grads, double *sumsq_dev);

/*
 * Multi-rank clip, part 2: the step of zero_shard_step with the clip
 * coefficient min(1, max_grad_norm / (sqrt(*global_sumsq_dev) + 1e-6)) taken
 * from a device double.  max_grad_norm must be > 0.  Never waits.
 */
int zero_shard_step_global_norm(zs_ctx *ctx, const void *const *grads, float lr, float beta1,
                                float beta2, float eps, float weight_decay, int64_t step,
                                float max_grad_norm, const double *global_sumsq_dev);

/*
 * Checkpoint / resharding.  The canonical state is every tensor's fp32 values
 * contiguous and unpadded, tensors in forward order (sum of numel elements per
 * array) -- independent of world_size, rank and bucket layout.  Saving it and
 * the step count is a checkpoint; exporting from N contexts and importing into
 * N' contexts of another plan over the same tensor list reshards (ZeRO shards
 * must be merged to resume on another card count: CS324 notes, exercise 11).
 * Each rank touches only the elements it owns; over all ranks of a plan the
 * pieces cover the canonical arrays exactly once.
 *
 * export: copies this rank's master, exp_avg, exp_avg_sq into the canonical
 *   device arrays.  import: the reverse, and also writes the param copy
 *   (bf16_rne(master), or fp16 for a ZS_FP16 context) for the imported
 *   elements; padding is not touched.
 * Canonical pointers are device pointers to sum(numel) floats each (may be
 * NULL only when the model is empty).  Enqueued on the context's stream.
 * Errors: ZS_EINVAL, ZS_EHIP.
 */
int zero_shard_export_state(zs_ctx *ctx, float *canon_master, float *canon_exp_avg,
                            float *canon_exp_avg_sq);
int zero_shard_import_state(zs_ctx *ctx, const float *canon_master, const float *canon_exp_avg,
                            const float *canon_exp_avg_sq);

/*
 * fp16 training with dynamic loss scaling (a context created with ZS_FP16:
 * grads[j] and the param buffer hold fp16).  The pages name fp16 overflow and
 * a loss scaler that must keep up as the hazard of 16-bit training (CS324
 * notes §13; 大模型基础设施工程 06, §12 pitfall 7); the scaler here is the usual
 * one (torch's GradScaler):
 *   g = ((sum_j grad_j) / M) * inv_scale,  inv_scale = fp32(1/scale)
 *   found_inf = the fp64 sum of g^2 is not finite (some g is NaN or Inf)
 *   found_inf:  nothing is updated; scale *= backoff_factor; tracker = 0
 *   otherwise:  [clip on the unscaled norm] the AdamW step at
 *               t = applied_steps + 1, param = fp16_rne(master);
 *               applied_steps += 1; after growth_interval such steps in a row
 *               tracker = 0 and scale *= growth_factor, unless the grown
 *               scale would be Inf (then the scale stays).
 * Everything, including the bias-correction constants for t, is decided on
 * the device: no host round trip per step.  zero_shard_amp_state_init enqueues
 * the initial state {init_scale, 0, 0}.  grad_norm_out (optional, waits)
 * receives the unscaled norm; ZS_NONFINITE then reports found_inf.
 * Errors: ZS_EINVAL, ZS_ESTATE (context without ZS_FP16), ZS_EHIP.
 */
int zero_shard_amp_state_init(zs_ctx *ctx, zs_amp_state *state_dev, float init_scale);
int zero_shard_step_amp(zs_ctx *ctx, const void *const *grads, float lr, float beta1, float beta2,
                        float eps, float weight_decay, float max_grad_norm,
                        zs_amp_state *state_dev, float growth_factor, float backoff_factor,
                        int32_t growth_interval, double *grad_norm_out);

/*
 * Multi-rank loss-scaled step.  With N > 1 every rank must take the same
 * skip decision, clip coefficient and scaler update, so they come from the sum
 * of g^2 over all shards: the norm over the whole model that clipping uses
 * (CS324 notes §7.4) and the overflow check of the scaler (CS324 notes §13).
 *
 * Part 1 enqueues sum_i g_i^2 (fp64, g unscaled with the scale in *state_dev;
 * NaN or Inf when some g is) of this shard into *sumsq_dev (an 8-byte-aligned
 * device double); with ZS_STAGE_AVERAGE it also stages the averages for part 2.
 * The caller sums these values over the ranks (a scalar all-reduce) and passes
 * the global sum to part 2, which runs zero_shard_step_amp's decision, scaler
 * update and step from it.  Each rank keeps its own copy of the scaler state;
 * the copies stay equal because every rank applies the same global value.  An
 * empty shard still takes part in both parts (part 1 writes 0).  Part 2 uses
 * the same grads as part 1 (or, with ZS_STAGE_AVERAGE, what part 1 staged).
 * Never waits.  Errors: ZS_EINVAL, ZS_ESTATE (context without ZS_FP16), ZS_EHIP.
 */
int zero_shard_grad_sumsq_amp(zs_ctx *ctx, const void *const *grads,
                              const zs_amp_state *state_dev, double *sumsq_dev);
int zero_shard_step_amp_global_norm(zs_ctx *ctx, const void *const *grads, float lr,
                                    float beta1, float beta2, float eps, float weight_decay,
                                    float max_grad_norm, zs_amp_state *state_dev,
                                    float growth_factor, float backoff_factor,
                                    int32_t growth_interval, const double *global_sumsq_dev);

/* ------------------------------------------- the step on host cores (offload) */

/*
 * Optimizer offload: the fp32 master, exp_avg and exp_avg_sq of the shard live
 * in host memory and host cores run the Adam step, so the GPU keeps only the
 * 16-bit params and gradients; the reduced gradient goes down and the params
 * come back over PCIe (大模型基础设施工程 06: §3.3 and §9.3 on ZeRO-Offload,
 * the optimizer offload to pinned CPU memory in the DeepSpeed configuration of
 * §11.3, FAQ Q5 on its throughput).  The arithmetic is the step's, operation
 * for operation, so results equal zero_shard_step's bit for bit.
 *
 * zs_host_adamw: the update alone, on host arrays of n elements holding shard
 *   elements [shard_off, shard_off + n) of the plan's shard: grad_avg is the
 *   averaged (M-way reduced) fp32 gradient, coef the clip coefficient (1 for
 *   none); master, exp_avg, exp_avg_sq are read and written, param receives
 *   bf16_rne(master), or fp16_rne(master) with flags = ZS_FP16 (flags: 0 or
 *   ZS_FP16).  Decay flags come from the plan.  n_threads host threads (0:
 *   every CPU this process may run on) are started for the call.
 *   Synchronous.  Errors: ZS_EINVAL, ZS_ENOMEM.
 */
int zs_host_adamw(const zs_plan *plan, int64_t shard_off, int64_t n, const float *grad_avg,
                  float coef, float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param,
                  float lr, float beta1, float beta2, float eps, float weight_decay,
                  int64_t step, int32_t n_threads, uint32_t flags);

typedef struct zs_offload zs_offload;

/* Pinned host staging a context needs for chunks of chunk_elems elements (a
 * positive multiple of 64), in bytes; 0 for an invalid chunk size. */
size_t zs_offload_staging_bytes(int64_t chunk_elems);

/*
 * Binds an offload context: param is device memory (shard_len bf16, or fp16
 * with ZS_FP16; written by every step); master, exp_avg, exp_avg_sq are host
 * memory (shard_len fp32
 * each; the caller initialises them as for zero_shard_init); workspace is device
 * memory of zs_workspace_bytes(plan, M, ZS_STAGE_AVERAGE) bytes, 256-byte
 * aligned; staging is pinned host memory (allocated pinned, e.g. hipHostMalloc)
 * of zs_offload_staging_bytes(chunk_elems) bytes, 256-byte aligned.  The
 * caller owns all of it.  n_threads host threads (0: every CPU this process may
 * run on) are started and kept until destroy; two copy streams at the default
 * priority are created.  flags: any of ZS_SKIP_NONFINITE, ZS_FP16 (fp16
 * gradients and param: zero_offload_step_amp), or 0.
 * Errors: ZS_EINVAL, ZS_ENOMEM, ZS_EHIP.
 */
int zero_offload_init(zs_offload **out, const zs_plan *plan, int32_t M, void *param,
                      float *master, float *exp_avg, float *exp_avg_sq, void *workspace,
                      size_t workspace_bytes, void *staging, size_t staging_bytes,
                      int64_t chunk_elems, int32_t n_threads, void *stream, uint32_t flags);

/*
 * One offloaded step, same arguments and results as zero_shard_step.  The norm
 * pass runs on the context's stream after the caller's earlier work; the
 * averages come to the host chunk by chunk while the host updates the previous
 * chunk and the one before goes back as bf16.  Returns when the host state is
 * updated; the param copies are still in flight, and later work on the
 * context's stream waits for them.  The norm is always available, so
 * grad_norm_out costs no extra wait.  On ZS_EHIP the host state may be
 * partly updated.  Errors: ZS_EINVAL, ZS_ESTATE (a ZS_FP16 context), ZS_EHIP.
 */
int zero_offload_step(zs_offload *ctx, const void *const *grads, float lr, float beta1,
                      float beta2, float eps, float weight_decay, int64_t step,
                      float max_grad_norm, double *grad_norm_out);

/*
 * The offloaded loss-scaled step (a context created with ZS_FP16): the scaler,
 * found-inf, the clip coefficient and the step constants at t = applied + 1 are
 * decided on the device exactly as in zero_shard_step_amp (same arguments, same
 * zs_amp_state); the host updates its fp32 state with those constants and the
 * fp16 param goes back.  A skipped step leaves the host state untouched.
 * Errors: ZS_EINVAL, ZS_ESTATE (context without ZS_FP16), ZS_EHIP.
 */
int zero_offload_step_amp(zs_offload *ctx, const void *const *grads, float lr, float beta1,
                          float beta2, float eps, float weight_decay, float max_grad_norm,
                          zs_amp_state *state_dev, float growth_factor, float backoff_factor,
                          int32_t growth_interval, double *grad_norm_out);

/*
 * Enqueues the initial scaler state {init_scale, 0, 0} into state_dev on the
 * offload context's device stream, as zero_shard_amp_state_init does for a
 * device context, so the first step on that stream reads it.
 * Errors: ZS_EINVAL (NULL or unaligned state_dev, init_scale not finite and
 * > 0), ZS_EHIP.
 */
int zero_offload_amp_state_init(zs_offload *ctx, zs_amp_state *state_dev, float init_scale);

/*
 * The multi-rank split of the offloaded steps, as for the device steps
 * (zero_shard_grad_sumsq / zero_shard_step_global_norm and their _amp twins):
 * part 1 runs the device norm pass, which also stages the averages part 2
 * sends to the host, and enqueues this shard's sum of squares into *sumsq_dev;
 * the caller sums it over the ranks; part 2 takes the clip coefficient (bf16:
 * max_grad_norm must be > 0), or the loss-scaled step's skip decision, clip and
 * scaler update, from the global value and runs the host update.  Part 1
 * enqueues only; part 2 returns when the host state is updated and the params
 * are queued back.  Part 2 uses what the same context's part 1 staged.
 * Errors: ZS_EINVAL, ZS_ESTATE (the wrong kind of context), ZS_EHIP.
 */
int zero_offload_grad_sumsq(zs_offload *ctx, const void *const *grads, double *sumsq_dev);
int zero_offload_step_global_norm(zs_offload *ctx, const void *const *grads, float lr,
                                  float beta1, float beta2, float eps, float weight_decay,
                                  int64_t step, float max_grad_norm,
                                  const double *global_sumsq_dev);
int zero_offload_grad_sumsq_amp(zs_offload *ctx, const void *const *grads,
                                const zs_amp_state *state_dev, double *sumsq_dev);
int zero_offload_step_amp_global_norm(zs_offload *ctx, const void *const *grads, float lr,
                                      float beta1, float beta2, float eps, float weight_decay,
                                      float max_grad_norm, zs_amp_state *state_dev,
                                      float growth_factor, float backoff_factor,
                                      int32_t growth_interval, const double *global_sumsq_dev);

/* Later offload steps enqueue their device work on `stream`. */
int zero_offload_set_stream(zs_offload *ctx, void *stream);

/* Waits for the context's copies, stops its threads and frees it. */
void zero_offload_destroy(zs_offload *ctx);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: one bf16
 * step of zero_shard_step's arithmetic (same kernels, same bits) on one rank's
 * buffers, with no context and no caller workspace.  The plan's run and
 * tile-flag tables, and for a clipped step the norm partials and the clip
 * scalars, go to a static device scratch of ZS_STATIC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends; the call
 * allocates nothing.  The scratch takes 16 B per decay run, 1 B per 1,024
 * elements when there is more than one run and, clipped, 1 B per 256 elements
 * of norm partials: a call that needs more (a clipped step beyond about 1.7G
 * elements, 2.1G with one run; an unclipped one beyond about 8.5G elements
 * with several runs) is refused with ZS_EINVAL and a message; use
 * zero_shard_init with a workspace then.
 *   plan        the layout (host), read during the call only: its run table
 *               travels to the scratch in kernel arguments and the tile flags
 *               are built from it on the device, so the call enqueues kernels
 *               only (no copy, no memset) and can be captured in a HIP graph
 *   M, buffers  as zero_shard_init / zero_shard_step (device pointers, 16-byte
 *               aligned, shard_len elements each); grads[0..M) bf16
 *   step, hyper-parameters, max_grad_norm: as zero_shard_step on a context
 *               made with flags 0 (bf16, no staged average, and a non-finite
 *               norm is not skipped); no norm output
 * Enqueues on `stream` and returns.  Every call on a GPU shares that GPU's
 * scratch (each call re-uploads its tables and writes every partial it reads,
 * so nothing needs clearing): calls that overlap on one GPU -- other threads,
 * other streams -- race and must be ordered by the caller; calls on one stream
 * are ordered already.  The first call on a device resolves the scratch's
 * address and queries the device: make it outside any graph capture (made
 * while `stream` is capturing, it is refused with ZS_EINVAL and leaves the
 * capture untouched).
 * Errors: ZS_EINVAL (found before anything is enqueued), ZS_EHIP.
 */
#define ZS_STATIC_SCRATCH_BYTES (8u << 20)
int zero_shard_step_static(const zs_plan *plan, int32_t M, void *param_bf16, float *master,
                           float *exp_avg, float *exp_avg_sq, const void *const *grads,
                           float lr, float beta1, float beta2, float eps, float weight_decay,
                           int64_t step, float max_grad_norm, void *stream);

/* The bf16 parameter shard and its length: after a step it holds the rank's
 * updated parameters, the buffer ZeRO-1's all-gather sends so that every rank
 * again holds the whole model (Lecture04 notes, "ZeRO-1"; CS336 第七讲
 * summary, Q2).  Host call, enqueues nothing. */
int zero_shard_params(zs_ctx *ctx, const void **param_bf16, int64_t *shard_len);

/* Later calls enqueue on `stream`. */
int zero_shard_set_stream(zs_ctx *ctx, void *stream);

/* Releases the context (host memory only; device buffers stay the caller's).
 * Like zero_shard_init, the library's own call: the pages define no interface
 * for it.  Work already enqueued is not waited for. */
void zero_shard_destroy(zs_ctx *ctx);

/* Message of the last failing call on this thread ("" if none). */
const char *zero_shard_last_error(void);

/* ------------------------------------------- optional device memory */

/*
 * For callers that want physically contiguous device memory for a large slab
 * (zs_slab_layout's); these are the library's only allocating calls, and no
 * other entry point uses them.  Measured on MI355X, the step on the Llama-70B
 * 1/16 shard (a 129 GB slab) ran 6.44 against 6.37 TB/s on ordinary device
 * memory as the first process on the device, but 6.15 against 6.25 after a
 * 108 GB process had run: where the contiguous range lands matters more than
 * its contiguity.  No default path uses it.
 *
 * zs_device_alloc_contiguous: `bytes` of device memory on `device`, physically
 * contiguous when the driver can provide it, else ordinary device memory (the
 * caller cannot tell which); NULL when neither is available.  `stream` is
 * ignored.  zs_device_free releases such a pointer (NULL is ignored).  The
 * signatures are those of a torch pluggable allocator, so a torch memory pool
 * can serve tensors from it.  Neither touches the current device of the
 * calling thread.
 */
void *zs_device_alloc_contiguous(size_t bytes, int device, void *stream);
void zs_device_free(void *ptr, size_t bytes, int device, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ZEROSHARD_H */
