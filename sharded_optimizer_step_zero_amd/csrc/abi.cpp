// abi.cpp -- the extern "C" entry points of the shard step (see include/zeroshard.h).
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <stdlib.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "../../include/zeroshard.h"
#include "abi_internal.h"
#include "internal.h"
#include "lds.h"

namespace zs {

thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int64_t max_groups_from_env() {
  const char* env = getenv("ZS_MAX_GROUPS_PER_LAUNCH");
  if (!env || !*env) return 0;
  const long long v = strtoll(env, nullptr, 10);
  return v > 0 ? (int64_t)v : 0;
}

}  // namespace zs

struct zs_ctx {
  int32_t M = 0;
  uint32_t flags = 0;
  bool fp16 = false;
  bool stage = false;  // ZS_STAGE_AVERAGE
  int64_t shard_len = 0, n_pieces = 0, n_whole_pieces = 0, canon_len = 0;
  int32_t n_runs = 0;
  zs::LdsPlan lds{};       // the dynamic LDS of every capped launch (lds.h)
  int64_t max_groups = 0;  // work-groups per launch slice (0: the dispatch limit)
  uint16_t* param = nullptr;
  float* master = nullptr;
  float* m = nullptr;
  float* v = nullptr;
  char* ws = nullptr;
  zs::WorkspaceLayout lay{};
  hipStream_t stream = nullptr;
};

namespace {

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// The scalars block is 256 bytes: ClipScalars at 0, the device-computed
// StepConsts at 64.  The staging area (ZS_STAGE_AVERAGE) comes first.
zs::WorkspaceLayout workspace_layout(int64_t shard_len, int64_t n_runs, int64_t n_pieces,
                                     int64_t n_partials, int64_t stage_elems) {
  static_assert(sizeof(zs::ClipScalars) <= 64 && sizeof(zs::StepConsts) <= 192,
                "scalars block overflow");
  zs::WorkspaceLayout l{};
  // the staged averages first, so that they start where the workspace starts
  // (zs_slab_layout staggers that start against the other streamed arrays)
  l.stage_off = 0;
  l.stage_bytes = round256((size_t)stage_elems * sizeof(float));
  l.runs_off = l.stage_bytes;
  l.runs_bytes = (size_t)(n_runs + 1) * sizeof(zs::Run);
  l.tflags_off = l.runs_off + round256(l.runs_bytes);
  l.tflags_bytes = (size_t)zs::tile_flag_words(shard_len, n_runs) * sizeof(uint32_t);
  l.pieces_off = l.tflags_off + round256(l.tflags_bytes);
  l.pieces_bytes = (size_t)n_pieces * sizeof(zs::Piece);
  l.partials_off = l.pieces_off + round256(l.pieces_bytes);
  l.scalars_off = l.partials_off + round256((size_t)n_partials * sizeof(double));
  l.total = l.scalars_off + 256;
  return l;
}

}  // namespace

// Helpers the other ABI translation unit (offload.cpp) shares; abi_internal.h.
namespace zs {

WorkspaceLayout plan_workspace(const zs_plan* plan, uint32_t flags) {
  return workspace_layout(plan->shard_len, (int64_t)plan->run_table.size() - 1,
                          (int64_t)plan->pieces.size(), zs::sumsq_partials(plan->shard_len),
                          (flags & ZS_STAGE_AVERAGE) ? plan->shard_len : 0);
}

int einval(const char* msg) {
  zs::set_error(msg);
  return ZS_EINVAL;
}

int ehip(const char* where, hipError_t e) {
  zs::set_error(std::string(where) + ": " + hipGetErrorString(e));
  return ZS_EHIP;
}

int check_hparams(float lr, float beta1, float beta2, float eps, float wd, int64_t step) {
  if (!(isfinite(lr) && isfinite(beta1) && isfinite(beta2) && isfinite(eps) && isfinite(wd)))
    return einval("zero_shard_step: hyper-parameters must be finite");
  if (lr < 0.0f) return einval("zero_shard_step: lr must be >= 0");
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return einval("zero_shard_step: beta1 and beta2 must lie in [0, 1)");
  if (!(eps > 0.0f)) return einval("zero_shard_step: eps must be > 0");
  if (wd < 0.0f) return einval("zero_shard_step: weight_decay must be >= 0");
  if (step < 1) return einval("zero_shard_step: step is 1-based and must be >= 1");
  return ZS_OK;
}

int check_amp_args(const char* who, float lr, float beta1, float beta2, float eps,
                   float weight_decay, float max_grad_norm, const zs_amp_state* state_dev,
                   float growth_factor, float backoff_factor, int32_t growth_interval,
                   AmpParams* p) {
  const std::string w(who);
  int rc = check_hparams(lr, beta1, beta2, eps, weight_decay, 1);
  if (rc) return rc;
  if (isnan(max_grad_norm) || isinf(max_grad_norm))
    return einval((w + ": max_grad_norm must be finite").c_str());
  if (!state_dev || ((uintptr_t)state_dev & 15u))
    return einval((w + ": state_dev must be a 16-byte-aligned device pointer").c_str());
  if (!(growth_factor >= 1.0f) || isinf(growth_factor) || !(backoff_factor > 0.0f) ||
      !(backoff_factor <= 1.0f) || growth_interval < 1)
    return einval((w + ": need growth >= 1, 0 < backoff <= 1, interval >= 1").c_str());
  p->lr = lr;
  p->beta1 = beta1;
  p->beta2 = beta2;
  p->eps = eps;
  p->weight_decay = weight_decay;
  p->max_norm = max_grad_norm;
  p->growth = growth_factor;
  p->backoff = backoff_factor;
  p->interval = growth_interval;
  p->clip = max_grad_norm > 0.0f ? 1 : 0;
  return ZS_OK;
}

}  // namespace zs

using zs::check_hparams;
using zs::ehip;
using zs::einval;
using zs::plan_workspace;

static_assert(zs::kCapTileElems == zs::kStepTileElems, "the caps count the step kernels' tiles");

namespace zs {

// The context's LDS reservations for M contributions over a shard, from the
// current device's CU count and LDS sizes and ZS_WAVES_PER_CU (unset: the
// measured table; 0: no cap; 3..64: that cap), each checked with the largest
// static LDS of the kernels that take a reservation against the device's
// per-workgroup limit.  ZS_OK, ZS_EINVAL (a bad override, or a reservation that
// does not fit: nothing is launched) or ZS_EHIP (a failed device query).
int make_lds_plan(int32_t M, int64_t shard_len, const char* who, LdsPlan* out) {
  const std::string w(who);
  int32_t override_waves;
  if (!parse_waves_override(getenv("ZS_WAVES_PER_CU"), &override_waves))
    return einval((w + ": ZS_WAVES_PER_CU must be 0 (no cap) or 3..64").c_str());
  int dev = 0, n_cu = 0, per_cu = 0, per_wg = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&per_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return ehip((w + ": device query").c_str(), e);
  const size_t lds_cu = per_cu > 0 ? (size_t)per_cu : kLdsPerCuDefault;
  size_t static_lds = 0;
  if ((e = reserved_kernels_static_lds(M, &static_lds)) != hipSuccess)
    return ehip((w + ": kernel attributes").c_str(), e);
  const LdsPlan p = lds_plan(M, shard_len, n_cu > 0 ? n_cu : 256, lds_cu, override_waves);
  const size_t wg_limit = per_wg > 0 ? (size_t)per_wg : kLdsPerWorkgroupFallback;
  if (!lds_plan_fits(p, static_lds, wg_limit, lds_cu))
    return einval((w + ": an LDS reservation (step " + std::to_string(p.step) + ", staged step " +
                   std::to_string(p.step_staged) + ", staged norm " +
                   std::to_string(p.stage_norm) + ", copy " + std::to_string(p.copy) +
                   " bytes, plus " + std::to_string(static_lds) +
                   " static) exceeds the device's per-workgroup LDS limit of " +
                   std::to_string(wg_limit) + " bytes")
                      .c_str());
  *out = p;
  return ZS_OK;
}

}  // namespace zs

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

zs::StepConsts step_consts(float lr, float beta1, float beta2, float eps, float wd, int64_t t) {
  return zs::step_consts(lr, beta1, beta2, eps, wd, t);
}

int gather_grads(const zs_ctx* ctx, const void* const* grads, zs::GradPtrs* out) {
  if (!grads) return einval("zero_shard_step: grads is NULL");
  memset(out, 0, sizeof(*out));
  for (int j = 0; j < ctx->M; j++) {
    if (!grads[j] || !aligned16(grads[j]))
      return einval("zero_shard_step: every grads[j] must be a non-NULL 16-byte-aligned pointer");
    out->p[j] = static_cast<const uint16_t*>(grads[j]);
  }
  return ZS_OK;
}

zs::ClipScalars* scalars(zs_ctx* ctx) {
  return reinterpret_cast<zs::ClipScalars*>(ctx->ws + ctx->lay.scalars_off);
}
// device-computed step constants of the loss-scaled path (same 256-byte block)
zs::StepConsts* device_consts(zs_ctx* ctx) {
  return reinterpret_cast<zs::StepConsts*>(ctx->ws + ctx->lay.scalars_off + 64);
}
float* stage_area(zs_ctx* ctx) {
  return ctx->stage ? reinterpret_cast<float*>(ctx->ws + ctx->lay.stage_off) : nullptr;
}
double* partials(zs_ctx* ctx) { return reinterpret_cast<double*>(ctx->ws + ctx->lay.partials_off); }
// the level-2 partials the finalize step sums
const double* final_partials(zs_ctx* ctx) {
  return partials(ctx) + zs::level1_partials(ctx->shard_len);
}
zs::RunTable run_table(zs_ctx* ctx) {
  zs::RunTable rt;
  rt.runs = reinterpret_cast<const zs::Run*>(ctx->ws + ctx->lay.runs_off);
  rt.tile_flags = ctx->lay.tflags_bytes
                      ? reinterpret_cast<const uint32_t*>(ctx->ws + ctx->lay.tflags_off)
                      : nullptr;
  rt.n_runs = ctx->n_runs;
  return rt;
}

}  // namespace

extern "C" size_t zs_workspace_bytes(const zs_plan* plan, int32_t M, uint32_t flags) {
  (void)M;
  if (!plan) return 0;
  return plan_workspace(plan, flags).total;
}

extern "C" int zs_slab_layout(const zs_plan* plan, int32_t M, uint32_t flags, int32_t n_grads,
                              size_t* offsets, size_t* slab_bytes) {
  if (!plan || !offsets || !slab_bytes) return einval("zs_slab_layout: NULL argument");
  if (M < 1 || M > ZS_MAX_M) return einval("zs_slab_layout: M must lie in [1, 16]");
  if (n_grads < 0 || n_grads > M) return einval("zs_slab_layout: n_grads must lie in [0, M]");
  if (flags & ~(ZS_SKIP_NONFINITE | ZS_FP16 | ZS_STAGE_AVERAGE))
    return einval("zs_slab_layout: unknown flag");
  const uint64_t S = (uint64_t)plan->shard_len;
  if (S > (uint64_t(1) << 56)) return einval("zs_slab_layout: shard too large");
  constexpr uint64_t kPeriod = uint64_t(1) << 21;  // 2 MiB
  constexpr uint64_t kStagger = uint64_t(1) << 12;  // 4 KiB
  const int32_t count = 5 + n_grads;
  uint64_t pos = 0;
  for (int32_t i = 0; i < count; i++) {
    uint64_t bytes;
    if (i == 0) bytes = 2 * S;                       // param (16-bit)
    else if (i <= 3) bytes = 4 * S;                  // master, exp_avg, exp_avg_sq
    else if (i < 4 + n_grads) bytes = 2 * S;         // gradient contributions
    else bytes = plan_workspace(plan, flags).total;  // workspace (staged averages first)
    pos = (pos + kPeriod - 1) / kPeriod * kPeriod + (uint64_t)i * kStagger;
    offsets[i] = (size_t)pos;
    pos += bytes;
  }
  *slab_bytes = (size_t)pos;
  return ZS_OK;
}

extern "C" int zero_shard_init(zs_ctx** out, const zs_plan* plan, int32_t M, void* param_bf16,
                               float* master, float* exp_avg, float* exp_avg_sq, void* workspace,
                               size_t workspace_bytes, void* stream, uint32_t flags) {
  if (!out) return einval("zero_shard_init: out is NULL");
  *out = nullptr;
  if (!plan) return einval("zero_shard_init: plan is NULL");
  if (M < 1 || M > ZS_MAX_M) return einval("zero_shard_init: M must lie in [1, 16]");
  if (flags & ~(ZS_SKIP_NONFINITE | ZS_FP16 | ZS_STAGE_AVERAGE))
    return einval("zero_shard_init: unknown flag");
  if (!param_bf16 || !master || !exp_avg || !exp_avg_sq || !workspace)
    return einval("zero_shard_init: NULL buffer");
  if (!aligned16(param_bf16) || !aligned16(master) || !aligned16(exp_avg) ||
      !aligned16(exp_avg_sq))
    return einval("zero_shard_init: buffers must be 16-byte aligned");
  if (((uintptr_t)workspace & 255u) != 0)
    return einval("zero_shard_init: workspace must be 256-byte aligned");
  if (plan->runs.size() > 0x3fffffff) return einval("zero_shard_init: too many runs");
  const zs::WorkspaceLayout lay = plan_workspace(plan, flags);
  if (workspace_bytes < lay.total)
    return einval("zero_shard_init: workspace smaller than zs_workspace_bytes(plan, M, flags)");
  const std::vector<zs::Run>& table = plan->run_table;  // runs + sentinel
  const std::vector<uint32_t>& tflags = plan->tile_flags;

  zs_ctx* c = new (std::nothrow) zs_ctx;
  if (!c) {
    zs::set_error("zero_shard_init: out of host memory");
    return ZS_ENOMEM;
  }
  c->M = M;
  c->flags = flags;
  c->fp16 = (flags & ZS_FP16) != 0;
  c->stage = (flags & ZS_STAGE_AVERAGE) != 0;
  c->shard_len = plan->shard_len;
  c->n_runs = (int32_t)(table.size() - 1);
  c->n_pieces = (int64_t)plan->pieces.size();
  c->n_whole_pieces = plan->n_whole_pieces;
  c->canon_len = plan->total_params;
  if (int rc = zs::make_lds_plan(M, plan->shard_len, "zero_shard_init", &c->lds)) {
    delete c;
    return rc;
  }
  c->max_groups = zs::max_groups_from_env();
  c->param = static_cast<uint16_t*>(param_bf16);
  c->master = master;
  c->m = exp_avg;
  c->v = exp_avg_sq;
  c->ws = static_cast<char*>(workspace);
  c->lay = lay;
  c->stream = static_cast<hipStream_t>(stream);
  {
    hipError_t e = hipMemcpyAsync(c->ws + lay.runs_off, table.data(),
                                  table.size() * sizeof(zs::Run), hipMemcpyHostToDevice,
                                  c->stream);
    if (e == hipSuccess && lay.tflags_bytes)
      e = hipMemcpyAsync(c->ws + lay.tflags_off, tflags.data(), lay.tflags_bytes,
                         hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess && lay.pieces_bytes)
      e = hipMemcpyAsync(c->ws + lay.pieces_off, plan->pieces.data(), lay.pieces_bytes,
                         hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
      delete c;
      return ehip("zero_shard_init: table upload", e);
    }
  }
  *out = c;
  return ZS_OK;
}

namespace {

// The norm pass (when needed) and the fused step, enqueued on ctx->stream.
int enqueue_step(zs_ctx* ctx, const zs::GradPtrs& g, const zs::StepConsts& k, bool need_norm,
                 bool clip, float max_norm, const double* external_sumsq) {
  hipError_t e;
  zs::ClipScalars* sc = scalars(ctx);
  // staging pays only where this call runs the norm pass itself
  float* stage = (need_norm && !external_sumsq) ? stage_area(ctx) : nullptr;
  if (need_norm) {
    if (!external_sumsq) {
      e = zs::launch_sumsq(ctx->M, g, ctx->shard_len, partials(ctx), stage, ctx->lds.stage_norm,
                           ctx->max_groups, ctx->stream);
      if (e != hipSuccess) return ehip("zero_shard_step: norm pass", e);
    }
    e = zs::launch_finalize(final_partials(ctx), zs::final_partials(ctx->shard_len),
                            external_sumsq, max_norm, clip ? 1 : 0,
                            (ctx->flags & ZS_SKIP_NONFINITE) ? 1 : 0, sc, ctx->stream);
    if (e != hipSuccess) return ehip("zero_shard_step: norm finalize", e);
  }
  if (stage)
    e = zs::launch_step_staged(false, stage, ctx->master, ctx->m, ctx->v, ctx->param,
                               ctx->shard_len, run_table(ctx), sc, k, nullptr,
                               ctx->lds.step_staged, ctx->max_groups, ctx->stream);
  else
    e = zs::launch_step(ctx->M, need_norm, g, ctx->master, ctx->m, ctx->v, ctx->param,
                        ctx->shard_len, run_table(ctx), sc, k, ctx->lds.step,
                        ctx->max_groups, ctx->stream);
  if (e != hipSuccess) return ehip("zero_shard_step: step kernel", e);
  return ZS_OK;
}

}  // namespace

int estate(const char* msg) {
  zs::set_error(msg);
  return ZS_ESTATE;
}

extern "C" int zero_shard_step(zs_ctx* ctx, const void* const* grads, float lr, float beta1,
                               float beta2, float eps, float weight_decay, int64_t step,
                               float max_grad_norm, double* grad_norm_out) {
  if (!ctx) return einval("zero_shard_step: ctx is NULL");
  if (ctx->fp16) return estate("zero_shard_step: fp16 context: use zero_shard_step_amp");
  int rc = check_hparams(lr, beta1, beta2, eps, weight_decay, step);
  if (rc) return rc;
  if (isnan(max_grad_norm) || isinf(max_grad_norm))
    return einval("zero_shard_step: max_grad_norm must be finite");
  zs::GradPtrs g;
  if ((rc = gather_grads(ctx, grads, &g))) return rc;
  if (ctx->shard_len == 0) {
    if (grad_norm_out) *grad_norm_out = 0.0;
    return ZS_OK;
  }
  const bool clip = max_grad_norm > 0.0f;
  const bool need_norm = clip || grad_norm_out || (ctx->flags & ZS_SKIP_NONFINITE);
  const zs::StepConsts k = step_consts(lr, beta1, beta2, eps, weight_decay, step);
  if ((rc = enqueue_step(ctx, g, k, need_norm, clip, max_grad_norm, nullptr))) return rc;
  if (grad_norm_out) {
    double norm = 0.0;
    hipError_t e = hipMemcpyAsync(&norm, &scalars(ctx)->norm, sizeof(double),
                                  hipMemcpyDeviceToHost, ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return ehip("zero_shard_step: reading the norm", e);
    *grad_norm_out = norm;
    if (!isfinite(norm)) return ZS_NONFINITE;
  }
  return ZS_OK;
}

extern "C" int zero_shard_grad_sumsq(zs_ctx* ctx, const void* const* grads, double* sumsq_dev) {
  if (!ctx) return einval("zero_shard_grad_sumsq: ctx is NULL");
  if (ctx->fp16) return estate("zero_shard_grad_sumsq: not available on an fp16 context");
  if (!sumsq_dev || ((uintptr_t)sumsq_dev & 7u))
    return einval("zero_shard_grad_sumsq: sumsq_dev must be an 8-byte-aligned device pointer");
  zs::GradPtrs g;
  int rc = gather_grads(ctx, grads, &g);
  if (rc) return rc;
  // an empty shard sums zero partials, which writes 0 (no memset: capture-safe)
  const int32_t n_final = ctx->shard_len ? zs::final_partials(ctx->shard_len) : 0;
  hipError_t e = hipSuccess;
  if (n_final)
    e = zs::launch_sumsq(ctx->M, g, ctx->shard_len, partials(ctx), nullptr, 0, ctx->max_groups,
                         ctx->stream);
  if (e == hipSuccess) e = zs::launch_sumsq_total(final_partials(ctx), n_final, sumsq_dev,
                                                  ctx->stream);
  return e == hipSuccess ? ZS_OK : ehip("zero_shard_grad_sumsq", e);
}

extern "C" int zero_shard_step_global_norm(zs_ctx* ctx, const void* const* grads, float lr,
                                           float beta1, float beta2, float eps,
                                           float weight_decay, int64_t step, float max_grad_norm,
                                           const double* global_sumsq_dev) {
  if (!ctx) return einval("zero_shard_step_global_norm: ctx is NULL");
  if (ctx->fp16) return estate("zero_shard_step_global_norm: not available on an fp16 context");
  int rc = check_hparams(lr, beta1, beta2, eps, weight_decay, step);
  if (rc) return rc;
  if (!(max_grad_norm > 0.0f) || isinf(max_grad_norm))
    return einval("zero_shard_step_global_norm: max_grad_norm must be finite and > 0");
  if (!global_sumsq_dev || ((uintptr_t)global_sumsq_dev & 7u))
    return einval("zero_shard_step_global_norm: global_sumsq_dev must be an aligned device pointer");
  zs::GradPtrs g;
  if ((rc = gather_grads(ctx, grads, &g))) return rc;
  if (ctx->shard_len == 0) return ZS_OK;
  const zs::StepConsts k = step_consts(lr, beta1, beta2, eps, weight_decay, step);
  return enqueue_step(ctx, g, k, true, true, max_grad_norm, global_sumsq_dev);
}

namespace {

int state_copy(zs_ctx* ctx, bool do_export, float* cm, float* cmm, float* cv, const char* who) {
  if (!ctx) return einval((std::string(who) + ": ctx is NULL").c_str());
  if (ctx->canon_len > 0 && (!cm || !cmm || !cv))
    return einval((std::string(who) + ": canonical buffers must be non-NULL").c_str());
  const hipError_t e = zs::launch_state_copy(
      do_export, ctx->fp16, reinterpret_cast<const zs::Piece*>(ctx->ws + ctx->lay.pieces_off),
      ctx->n_pieces, ctx->n_whole_pieces, ctx->master, ctx->m, ctx->v, ctx->param, cm, cmm, cv,
      ctx->lds.copy, ctx->max_groups, ctx->stream);
  return e == hipSuccess ? ZS_OK : ehip(who, e);
}

}  // namespace

extern "C" int zero_shard_export_state(zs_ctx* ctx, float* canon_master, float* canon_exp_avg,
                                       float* canon_exp_avg_sq) {
  return state_copy(ctx, true, canon_master, canon_exp_avg, canon_exp_avg_sq,
                    "zero_shard_export_state");
}

extern "C" int zero_shard_import_state(zs_ctx* ctx, const float* canon_master,
                                       const float* canon_exp_avg,
                                       const float* canon_exp_avg_sq) {
  return state_copy(ctx, false, const_cast<float*>(canon_master), const_cast<float*>(canon_exp_avg),
                    const_cast<float*>(canon_exp_avg_sq), "zero_shard_import_state");
}

extern "C" int zero_shard_amp_state_init(zs_ctx* ctx, zs_amp_state* state_dev, float init_scale) {
  if (!ctx) return einval("zero_shard_amp_state_init: ctx is NULL");
  if (!state_dev || ((uintptr_t)state_dev & 15u))
    return einval("zero_shard_amp_state_init: state_dev must be a 16-byte-aligned device pointer");
  if (!(init_scale > 0.0f) || isinf(init_scale))
    return einval("zero_shard_amp_state_init: init_scale must be finite and > 0");
  const hipError_t e = zs::launch_amp_state_init(reinterpret_cast<zs::AmpState*>(state_dev),
                                                 init_scale, ctx->stream);
  return e == hipSuccess ? ZS_OK : ehip("zero_shard_amp_state_init", e);
}

namespace {

// Argument checks of the loss-scaled steps; fills the finalize parameters.
int amp_args(const zs_ctx* ctx, const char* who, float lr, float beta1, float beta2, float eps,
             float weight_decay, float max_grad_norm, const zs_amp_state* state_dev,
             float growth_factor, float backoff_factor, int32_t growth_interval,
             zs::AmpParams* p) {
  const std::string w(who);
  if (!ctx) return einval((w + ": ctx is NULL").c_str());
  if (!ctx->fp16) return estate((w + ": needs a context created with ZS_FP16").c_str());
  return zs::check_amp_args(who, lr, beta1, beta2, eps, weight_decay, max_grad_norm, state_dev,
                            growth_factor, backoff_factor, growth_interval, p);
}

// The rest of a loss-scaled step once the norm pass has run (or, with
// external, once the global sum of squares is known): the finalize (skip,
// clip coefficient, scaler update, step constants) and the step kernel.  An
// empty shard still runs the finalize, so its scaler advances like the others.
int amp_finish(zs_ctx* ctx, const zs::GradPtrs& g, zs::AmpState* st, const zs::AmpParams& p,
               const double* external, double* grad_norm_out, const char* who) {
  const std::string w(who);
  const int32_t n_final = ctx->shard_len ? zs::final_partials(ctx->shard_len) : 0;
  hipError_t e = zs::launch_amp_finalize(final_partials(ctx), n_final, external, st, p,
                                         scalars(ctx), device_consts(ctx), ctx->stream);
  if (e != hipSuccess) return ehip((w + ": finalize").c_str(), e);
  if (ctx->shard_len > 0) {
    if (ctx->stage)
      e = zs::launch_step_staged(true, stage_area(ctx), ctx->master, ctx->m, ctx->v, ctx->param,
                                 ctx->shard_len, run_table(ctx), scalars(ctx),
                                 zs::StepConsts{}, device_consts(ctx),
                                 ctx->lds.step_staged, ctx->max_groups, ctx->stream);
    else
      e = zs::launch_step_f16(ctx->M, g, ctx->master, ctx->m, ctx->v, ctx->param,
                              ctx->shard_len, run_table(ctx), scalars(ctx), device_consts(ctx),
                              ctx->lds.step, ctx->max_groups, ctx->stream);
    if (e != hipSuccess) return ehip((w + ": step kernel").c_str(), e);
  }
  if (grad_norm_out) {
    double norm = 0.0;
    e = hipMemcpyAsync(&norm, &scalars(ctx)->norm, sizeof(double), hipMemcpyDeviceToHost,
                       ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return ehip((w + ": reading the norm").c_str(), e);
    *grad_norm_out = norm;
    if (!isfinite(norm)) return ZS_NONFINITE;
  }
  return ZS_OK;
}

}  // namespace

extern "C" int zero_shard_step_amp(zs_ctx* ctx, const void* const* grads, float lr, float beta1,
                                   float beta2, float eps, float weight_decay,
                                   float max_grad_norm, zs_amp_state* state_dev,
                                   float growth_factor, float backoff_factor,
                                   int32_t growth_interval, double* grad_norm_out) {
  const char* who = "zero_shard_step_amp";
  zs::AmpParams p;
  int rc = amp_args(ctx, who, lr, beta1, beta2, eps, weight_decay, max_grad_norm, state_dev,
                    growth_factor, backoff_factor, growth_interval, &p);
  if (rc) return rc;
  zs::GradPtrs g;
  if ((rc = gather_grads(ctx, grads, &g))) return rc;
  zs::AmpState* st = reinterpret_cast<zs::AmpState*>(state_dev);
  if (ctx->shard_len > 0) {
    const hipError_t e =
        zs::launch_sumsq_f16(ctx->M, g, ctx->shard_len, partials(ctx), st, stage_area(ctx),
                             ctx->lds.stage_norm, ctx->max_groups, ctx->stream);
    if (e != hipSuccess) return ehip("zero_shard_step_amp: norm pass", e);
  }
  return amp_finish(ctx, g, st, p, nullptr, grad_norm_out, who);
}

extern "C" int zero_shard_grad_sumsq_amp(zs_ctx* ctx, const void* const* grads,
                                         const zs_amp_state* state_dev, double* sumsq_dev) {
  if (!ctx) return einval("zero_shard_grad_sumsq_amp: ctx is NULL");
  if (!ctx->fp16)
    return estate("zero_shard_grad_sumsq_amp: needs a context created with ZS_FP16");
  if (!state_dev || ((uintptr_t)state_dev & 15u))
    return einval("zero_shard_grad_sumsq_amp: state_dev must be a 16-byte-aligned device pointer");
  if (!sumsq_dev || ((uintptr_t)sumsq_dev & 7u))
    return einval("zero_shard_grad_sumsq_amp: sumsq_dev must be an 8-byte-aligned device pointer");
  zs::GradPtrs g;
  int rc = gather_grads(ctx, grads, &g);
  if (rc) return rc;
  const int32_t n_final = ctx->shard_len ? zs::final_partials(ctx->shard_len) : 0;
  hipError_t e = hipSuccess;
  if (n_final)
    e = zs::launch_sumsq_f16(ctx->M, g, ctx->shard_len, partials(ctx),
                             reinterpret_cast<const zs::AmpState*>(state_dev), stage_area(ctx),
                             ctx->lds.stage_norm, ctx->max_groups, ctx->stream);
  if (e == hipSuccess)
    e = zs::launch_sumsq_total(final_partials(ctx), n_final, sumsq_dev, ctx->stream);
  return e == hipSuccess ? ZS_OK : ehip("zero_shard_grad_sumsq_amp", e);
}

extern "C" int zero_shard_step_amp_global_norm(zs_ctx* ctx, const void* const* grads, float lr,
                                               float beta1, float beta2, float eps,
                                               float weight_decay, float max_grad_norm,
                                               zs_amp_state* state_dev, float growth_factor,
                                               float backoff_factor, int32_t growth_interval,
                                               const double* global_sumsq_dev) {
  const char* who = "zero_shard_step_amp_global_norm";
  zs::AmpParams p;
  int rc = amp_args(ctx, who, lr, beta1, beta2, eps, weight_decay, max_grad_norm, state_dev,
                    growth_factor, backoff_factor, growth_interval, &p);
  if (rc) return rc;
  if (!global_sumsq_dev || ((uintptr_t)global_sumsq_dev & 7u))
    return einval(
        "zero_shard_step_amp_global_norm: global_sumsq_dev must be an aligned device pointer");
  zs::GradPtrs g;
  if ((rc = gather_grads(ctx, grads, &g))) return rc;
  return amp_finish(ctx, g, reinterpret_cast<zs::AmpState*>(state_dev), p, global_sumsq_dev,
                    nullptr, who);
}

extern "C" int zero_shard_params(zs_ctx* ctx, const void** param_bf16, int64_t* shard_len) {
  if (!ctx) return einval("zero_shard_params: ctx is NULL");
  if (param_bf16) *param_bf16 = ctx->param;
  if (shard_len) *shard_len = ctx->shard_len;
  return ZS_OK;
}

extern "C" int zero_shard_set_stream(zs_ctx* ctx, void* stream) {
  if (!ctx) return einval("zero_shard_set_stream: ctx is NULL");
  ctx->stream = static_cast<hipStream_t>(stream);
  return ZS_OK;
}

extern "C" void zero_shard_destroy(zs_ctx* ctx) { delete ctx; }

extern "C" const char* zero_shard_last_error(void) { return zs::g_last_error.c_str(); }
