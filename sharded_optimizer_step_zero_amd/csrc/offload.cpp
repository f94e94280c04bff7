// offload.cpp -- the optimizer step on host cores with PCIe staging, and the
// host update alone (see include/zeroshard.h, "optimizer step on host cores").
//
// One step: the device's norm pass reduces the M contributions and stages each
// element's fp32 average in the workspace (and gives the norm and clip scalars);
// the averages come to pinned host memory chunk by chunk on one copy stream,
// host threads update the fp32 state in host memory, and each chunk's bf16
// params go back on a second copy stream, so the two PCIe directions and the
// host work overlap.  Two staging buffers per direction; the host waits only on
// events of its own copies.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <new>
#include <string>
#include <system_error>
#include <utility>
#include <vector>

#include "../../include/zeroshard.h"
#include "abi_internal.h"
#include "host.h"
#include "internal.h"

namespace {

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Pinned staging: 256 bytes for the clip scalars, two fp32 gradient buffers and
// two bf16 param buffers of chunk elements each.
struct StagingLayout {
  size_t g_off[2], p_off[2], total;
};

StagingLayout staging_layout(int64_t chunk) {
  StagingLayout s{};
  size_t off = 256;
  for (int b = 0; b < 2; b++) {
    s.g_off[b] = off;
    off += round256((size_t)chunk * sizeof(float));
  }
  for (int b = 0; b < 2; b++) {
    s.p_off[b] = off;
    off += round256((size_t)chunk * sizeof(uint16_t));
  }
  s.total = off;
  return s;
}

zs::HostConsts host_consts(const zs::StepConsts& k) {
  zs::HostConsts h;
  h.beta1 = k.beta1;
  h.beta2 = k.beta2;
  h.c1 = k.c1;
  h.c2 = k.c2;
  h.alpha = k.alpha;
  h.bhat = k.bhat;
  h.eps = k.eps;
  h.decay_mul = k.decay_mul;
  return h;
}

// The plan's runs followed by a sentinel at the shard length.
std::vector<zs::HostRun> host_runs(const zs_plan* plan) {
  std::vector<zs::HostRun> t;
  t.reserve(plan->runs.size() + 2);
  for (const zs::Run& r : plan->runs) t.push_back({r.start, r.flags, 0});
  if (t.empty()) t.push_back({0, 0, 0});
  t.push_back({plan->shard_len, 0, 0});
  return t;
}

// The pipeline's chunks (offset, length): they start at chunk/8 and double up to
// chunk, and the tail is halved down again, so the host starts after a short
// first copy and the last copy back is short too.  Lengths are multiples of 64
// except the shard's own ragged end.
std::vector<std::pair<int64_t, int64_t>> chunk_schedule(int64_t S, int64_t chunk) {
  std::vector<std::pair<int64_t, int64_t>> out;
  const int64_t small = std::max<int64_t>(64, chunk / 8 / 64 * 64);
  int64_t off = 0, ramp = std::min(small, chunk);
  while (off < S) {
    const int64_t r = S - off;
    int64_t len;
    if (r <= small) {
      len = r;
    } else if (r <= 2 * chunk) {
      len = std::max(small, (r / 2 + 63) / 64 * 64);  // halve the tail
    } else {
      len = ramp;
      ramp = std::min(2 * ramp, chunk);  // stops at chunk: no overflow however many chunks
    }
    out.emplace_back(off, len);
    off += len;
  }
  return out;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int enomem(const char* msg) {
  zs::set_error(msg);
  return ZS_ENOMEM;
}

}  // namespace

struct zs_offload {
  int32_t M = 0;
  uint32_t flags = 0;
  bool fp16 = false;  // ZS_FP16: fp16 gradients and param, zero_offload_step_amp
  int64_t shard_len = 0, chunk = 0;
  int64_t max_groups = 0;  // work-groups per launch slice (0: the dispatch limit)
  zs::LdsPlan lds{};       // the dynamic LDS of every capped launch (lds.h)
  std::vector<zs::HostRun> runs;
  std::vector<std::pair<int64_t, int64_t>> chunks;
  uint16_t* param = nullptr;
  float* master = nullptr;
  float* m = nullptr;
  float* v = nullptr;
  char* ws = nullptr;
  zs::WorkspaceLayout lay{};
  char* staging = nullptr;
  StagingLayout sl{};
  hipStream_t stream = nullptr, d2h = nullptr, h2d = nullptr;
  hipEvent_t ready = nullptr, scalars = nullptr, done = nullptr;
  hipEvent_t g_ready[2] = {nullptr, nullptr}, p_sent[2] = {nullptr, nullptr};
  std::vector<hipEvent_t> chunk_done;  // per chunk: its averages are staged on the device
  std::unique_ptr<zs::HostPool> pool;

  ~zs_offload() {
    // teardown: nothing left to report an error to
    if (d2h) (void)hipStreamSynchronize(d2h);
    if (h2d) (void)hipStreamSynchronize(h2d);
    for (hipEvent_t e : {ready, scalars, done, g_ready[0], g_ready[1], p_sent[0], p_sent[1]})
      if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : chunk_done)
      if (e) (void)hipEventDestroy(e);
    if (d2h) (void)hipStreamDestroy(d2h);
    if (h2d) (void)hipStreamDestroy(h2d);
  }
};

extern "C" size_t zs_offload_staging_bytes(int64_t chunk_elems) {
  if (chunk_elems < 64 || chunk_elems % 64) return 0;
  return staging_layout(chunk_elems).total;
}

extern "C" int zero_offload_init(zs_offload** out, const zs_plan* plan, int32_t M, void* param,
                                 float* master, float* exp_avg, float* exp_avg_sq, void* workspace,
                                 size_t workspace_bytes, void* staging, size_t staging_bytes,
                                 int64_t chunk_elems, int32_t n_threads, void* stream,
                                 uint32_t flags) {
  using zs::einval;
  if (!out) return einval("zero_offload_init: out is NULL");
  *out = nullptr;
  if (!plan) return einval("zero_offload_init: plan is NULL");
  if (M < 1 || M > ZS_MAX_M) return einval("zero_offload_init: M must lie in [1, 16]");
  if (flags & ~(ZS_SKIP_NONFINITE | ZS_STAGE_AVERAGE | ZS_FP16))
    return einval("zero_offload_init: flags may hold ZS_SKIP_NONFINITE and ZS_FP16 "
                  "(staging is implied)");
  if (chunk_elems < 64 || chunk_elems % 64)
    return einval("zero_offload_init: chunk_elems must be a positive multiple of 64");
  if (n_threads < 0 || n_threads > 1024)
    return einval("zero_offload_init: n_threads must lie in [0, 1024]");
  if (!param || !master || !exp_avg || !exp_avg_sq || !workspace || !staging)
    return einval("zero_offload_init: NULL buffer");
  if (!aligned(param, 16) || !aligned(master, 16) || !aligned(exp_avg, 16) ||
      !aligned(exp_avg_sq, 16))
    return einval("zero_offload_init: buffers must be 16-byte aligned");
  if (!aligned(workspace, 256) || !aligned(staging, 256))
    return einval("zero_offload_init: workspace and staging must be 256-byte aligned");
  const zs::WorkspaceLayout lay = zs::plan_workspace(plan, flags | ZS_STAGE_AVERAGE);
  if (workspace_bytes < lay.total)
    return einval("zero_offload_init: workspace smaller than "
                  "zs_workspace_bytes(plan, M, ZS_STAGE_AVERAGE)");
  const StagingLayout sl = staging_layout(chunk_elems);
  if (staging_bytes < sl.total)
    return einval("zero_offload_init: staging smaller than zs_offload_staging_bytes(chunk_elems)");

  std::unique_ptr<zs_offload> c(new (std::nothrow) zs_offload);
  if (!c) return enomem("zero_offload_init: out of host memory");
  c->M = M;
  c->max_groups = zs::max_groups_from_env();
  if (int rc = zs::make_lds_plan(M, plan->shard_len, "zero_offload_init", &c->lds)) return rc;
  c->flags = flags;
  c->fp16 = (flags & ZS_FP16) != 0;
  c->shard_len = plan->shard_len;
  c->chunk = chunk_elems;
  c->param = static_cast<uint16_t*>(param);
  c->master = master;
  c->m = exp_avg;
  c->v = exp_avg_sq;
  c->ws = static_cast<char*>(workspace);
  c->lay = lay;
  c->staging = static_cast<char*>(staging);
  c->sl = sl;
  c->stream = static_cast<hipStream_t>(stream);
  try {
    c->runs = host_runs(plan);
    c->chunks = chunk_schedule(plan->shard_len, chunk_elems);
    c->chunk_done.assign(c->chunks.size(), nullptr);
    c->pool.reset(new zs::HostPool(n_threads > 0 ? n_threads : zs::default_host_threads()));
  } catch (const std::bad_alloc&) {
    return enomem("zero_offload_init: out of host memory");
  } catch (const std::system_error&) {
    return enomem("zero_offload_init: could not start the host threads");
  }
  // copy streams at the default priority; they order themselves against the
  // caller's stream through events
  hipError_t e = hipStreamCreateWithFlags(&c->d2h, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->h2d, hipStreamNonBlocking);
  for (hipEvent_t* ev : {&c->ready, &c->scalars, &c->done, &c->g_ready[0], &c->g_ready[1],
                         &c->p_sent[0], &c->p_sent[1]})
    if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
  for (hipEvent_t& ev : c->chunk_done)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  // both param buffers start out free: their events complete on an empty stream
  for (int b = 0; b < 2 && e == hipSuccess; b++) e = hipEventRecord(c->p_sent[b], c->h2d);
  if (e == hipSuccess) e = hipStreamSynchronize(c->h2d);
  if (e != hipSuccess) return zs::ehip("zero_offload_init: streams and events", e);
  *out = c.release();
  return ZS_OK;
}

namespace {

// After a failed HIP call inside a step: let the copies already queued finish
// (they target the staging buffers) before reporting.
int fail(zs_offload* c, const char* where, hipError_t e) {
  (void)hipStreamSynchronize(c->d2h);
  (void)hipStreamSynchronize(c->h2d);
  return zs::ehip(where, e);
}

}  // namespace

namespace {

int gather(const zs_offload* c, const void* const* grads, zs::GradPtrs* g, const char* who) {
  if (!grads) return zs::einval((std::string(who) + ": grads is NULL").c_str());
  memset(g, 0, sizeof *g);
  for (int j = 0; j < c->M; j++) {
    if (!grads[j] || !aligned(grads[j], 16))
      return zs::einval((std::string(who) +
                         ": every grads[j] must be a non-NULL 16-byte-aligned pointer")
                            .c_str());
    g->p[j] = static_cast<const uint16_t*>(grads[j]);
  }
  return ZS_OK;
}

// Everything after the device part of a step (norm pass and finalize, already
// queued on the caller's stream, which wrote the 256-byte scalars block and the
// staged averages): the scalars and the averages come to the host, the host
// updates chunk by chunk, the params go back.  k_host: the step constants, or
// null to take the ones the device computed (the loss-scaled step).
// per_chunk (non-null: a bf16 step that needs no norm): the device part has not
// run; it is queued here chunk by chunk, each chunk's copy to the host waiting
// only for its own averages, so the host starts on the first chunk while the
// device still reduces the rest.  The coefficient is then 1 and nothing skips.
int pipeline(zs_offload* c, const zs::HostConsts* k_host, bool out_f16, double* grad_norm_out,
             const char* who, const zs::GradPtrs* per_chunk = nullptr) {
  float* stage = reinterpret_cast<float*>(c->ws + c->lay.stage_off);
  const char* block_dev = c->ws + c->lay.scalars_off;
  volatile char* block_host = c->staging;  // the first 256 staging bytes
  // both copy streams start after everything the caller queued before this step
  hipError_t e = hipEventRecord(c->ready, c->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->d2h, c->ready, 0);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->h2d, c->ready, 0);
  if (per_chunk) {
    double* partials = reinterpret_cast<double*>(c->ws + c->lay.partials_off);
    for (size_t ci = 0; ci < c->chunks.size() && e == hipSuccess; ci++) {
      const int64_t off = c->chunks[ci].first, len = c->chunks[ci].second;
      zs::GradPtrs g = *per_chunk;
      for (int j = 0; j < c->M; j++) g.p[j] += off;
      e = zs::launch_sumsq(c->M, g, len, partials, stage + off, c->lds.stage_norm, c->max_groups,
                           c->stream);
      if (e == hipSuccess) e = hipEventRecord(c->chunk_done[ci], c->stream);
    }
  } else {
    if (e == hipSuccess)
      e = hipMemcpyAsync((void*)block_host, block_dev, 256, hipMemcpyDeviceToHost, c->d2h);
    if (e == hipSuccess) e = hipEventRecord(c->scalars, c->d2h);
  }
  if (e != hipSuccess) return fail(c, who, e);

  const int64_t n_chunks = (int64_t)c->chunks.size();
  auto gbuf = [&](int b) { return reinterpret_cast<float*>(c->staging + c->sl.g_off[b]); };
  auto pbuf = [&](int b) { return reinterpret_cast<uint16_t*>(c->staging + c->sl.p_off[b]); };
  auto fetch = [&](int64_t ci) {  // queue chunk ci's averages into gradient buffer ci % 2
    const int64_t off = c->chunks[ci].first, len = c->chunks[ci].second;
    const int b = (int)(ci & 1);
    hipError_t r = per_chunk ? hipStreamWaitEvent(c->d2h, c->chunk_done[ci], 0) : hipSuccess;
    if (r == hipSuccess)
      r = hipMemcpyAsync(gbuf(b), stage + off, (size_t)len * sizeof(float),
                         hipMemcpyDeviceToHost, c->d2h);
    if (r == hipSuccess) r = hipEventRecord(c->g_ready[b], c->d2h);
    return r;
  };
  for (int64_t ci = 0; ci < std::min<int64_t>(2, n_chunks) && e == hipSuccess; ci++) e = fetch(ci);
  if (e == hipSuccess && !per_chunk) e = hipEventSynchronize(c->scalars);
  if (e != hipSuccess) return fail(c, who, e);
  zs::ClipScalars sc{};
  zs::StepConsts kd{};
  if (per_chunk) {
    sc.coef = 1.0f;
  } else {
    memcpy(&sc, (const void*)block_host, sizeof sc);
    memcpy(&kd, (const void*)(block_host + 64), sizeof kd);
  }
  if (grad_norm_out) *grad_norm_out = sc.norm;
  const int done_rc = (grad_norm_out && !isfinite(sc.norm)) ? ZS_NONFINITE : ZS_OK;
  if (sc.skip) {  // the step is skipped: the state stays as it is
    e = hipStreamSynchronize(c->d2h);
    return e == hipSuccess ? done_rc : fail(c, who, e);
  }
  const zs::HostConsts k = k_host ? *k_host : host_consts(kd);

  const int32_t n_runs = (int32_t)c->runs.size() - 1;
  for (int64_t ci = 0; ci < n_chunks; ci++) {
    const int64_t off = c->chunks[ci].first, len = c->chunks[ci].second;
    const int b = (int)(ci & 1);
    e = hipEventSynchronize(c->g_ready[b]);           // this chunk's averages have landed
    if (e == hipSuccess) e = hipEventSynchronize(c->p_sent[b]);  // param buffer b is free again
    if (e != hipSuccess) return fail(c, who, e);
    zs::host_adamw(*c->pool, c->runs.data(), n_runs, off, len, gbuf(b), sc.coef, c->master + off,
                   c->m + off, c->v + off, pbuf(b), k, out_f16);
    if (ci + 2 < n_chunks) e = fetch(ci + 2);
    if (e == hipSuccess)
      e = hipMemcpyAsync(c->param + off, pbuf(b), (size_t)len * sizeof(uint16_t),
                         hipMemcpyHostToDevice, c->h2d);
    if (e == hipSuccess) e = hipEventRecord(c->p_sent[b], c->h2d);
    if (e != hipSuccess) return fail(c, who, e);
  }
  // later work on the caller's stream sees the new params
  e = hipEventRecord(c->done, c->h2d);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->stream, c->done, 0);
  if (e != hipSuccess) return fail(c, who, e);
  return done_rc;
}

int estate(const char* msg) {
  zs::set_error(msg);
  return ZS_ESTATE;
}

}  // namespace

extern "C" int zero_offload_step(zs_offload* c, const void* const* grads, float lr, float beta1,
                                 float beta2, float eps, float weight_decay, int64_t step,
                                 float max_grad_norm, double* grad_norm_out) {
  using zs::einval;
  if (!c) return einval("zero_offload_step: ctx is NULL");
  if (c->fp16) return estate("zero_offload_step: fp16 context: use zero_offload_step_amp");
  int rc = zs::check_hparams(lr, beta1, beta2, eps, weight_decay, step);
  if (rc) return rc;
  if (isnan(max_grad_norm) || isinf(max_grad_norm))
    return einval("zero_offload_step: max_grad_norm must be finite");
  zs::GradPtrs g;
  if ((rc = gather(c, grads, &g, "zero_offload_step"))) return rc;
  if (c->shard_len == 0) {
    if (grad_norm_out) *grad_norm_out = 0.0;
    return ZS_OK;
  }
  const int64_t S = c->shard_len;
  const zs::HostConsts k =
      host_consts(zs::step_consts(lr, beta1, beta2, eps, weight_decay, step));
  // nothing needs the norm: the device reduce runs chunk by chunk inside the pipeline
  if (!(max_grad_norm > 0.0f) && !(c->flags & ZS_SKIP_NONFINITE) && !grad_norm_out)
    return pipeline(c, &k, false, nullptr, "zero_offload_step", &g);
  float* stage = reinterpret_cast<float*>(c->ws + c->lay.stage_off);
  double* partials = reinterpret_cast<double*>(c->ws + c->lay.partials_off);
  zs::ClipScalars* sc_dev = reinterpret_cast<zs::ClipScalars*>(c->ws + c->lay.scalars_off);
  // the device part: reduce, stage the averages, norm and clip scalars
  hipError_t e =
      zs::launch_sumsq(c->M, g, S, partials, stage, c->lds.stage_norm, c->max_groups, c->stream);
  if (e == hipSuccess)
    e = zs::launch_finalize(partials + zs::level1_partials(S), zs::final_partials(S), nullptr,
                            max_grad_norm, max_grad_norm > 0.0f ? 1 : 0,
                            (c->flags & ZS_SKIP_NONFINITE) ? 1 : 0, sc_dev, c->stream);
  if (e != hipSuccess) return zs::ehip("zero_offload_step: norm pass", e);
  return pipeline(c, &k, false, grad_norm_out, "zero_offload_step");
}

extern "C" int zero_offload_step_amp(zs_offload* c, const void* const* grads, float lr,
                                     float beta1, float beta2, float eps, float weight_decay,
                                     float max_grad_norm, zs_amp_state* state_dev,
                                     float growth_factor, float backoff_factor,
                                     int32_t growth_interval, double* grad_norm_out) {
  const char* who = "zero_offload_step_amp";
  if (!c) return zs::einval("zero_offload_step_amp: ctx is NULL");
  if (!c->fp16) return estate("zero_offload_step_amp: needs a context created with ZS_FP16");
  zs::AmpParams p;
  int rc = zs::check_amp_args(who, lr, beta1, beta2, eps, weight_decay, max_grad_norm, state_dev,
                              growth_factor, backoff_factor, growth_interval, &p);
  if (rc) return rc;
  zs::GradPtrs g;
  if ((rc = gather(c, grads, &g, who))) return rc;
  const int64_t S = c->shard_len;
  zs::AmpState* st = reinterpret_cast<zs::AmpState*>(state_dev);
  float* stage = reinterpret_cast<float*>(c->ws + c->lay.stage_off);
  double* partials = reinterpret_cast<double*>(c->ws + c->lay.partials_off);
  char* block = c->ws + c->lay.scalars_off;
  // the device part: unscaled averages staged, found-inf, scaler update and the
  // step constants at t = applied + 1, all on the device; an empty shard still
  // runs the finalize, so its scaler advances like every other rank's
  hipError_t e = hipSuccess;
  if (S > 0)
    e = zs::launch_sumsq_f16(c->M, g, S, partials, st, stage, c->lds.stage_norm, c->max_groups,
                             c->stream);
  if (e == hipSuccess)
    e = zs::launch_amp_finalize(partials + zs::level1_partials(S),
                                S ? zs::final_partials(S) : 0, nullptr, st, p,
                                reinterpret_cast<zs::ClipScalars*>(block),
                                reinterpret_cast<zs::StepConsts*>(block + 64), c->stream);
  if (e != hipSuccess) return zs::ehip("zero_offload_step_amp: norm pass", e);
  return pipeline(c, nullptr, true, grad_norm_out, who);
}

namespace {

// Part 1 of the multi-rank split on an offload context: the device norm pass
// (which stages the averages part 2 sends to the host) and this shard's sum of
// squares into *sumsq_dev.
int offload_sumsq(zs_offload* c, const void* const* grads, const zs_amp_state* state_dev,
                  double* sumsq_dev, const char* who) {
  const std::string w(who);
  if (!sumsq_dev || !aligned(sumsq_dev, 8))
    return zs::einval((w + ": sumsq_dev must be an 8-byte-aligned device pointer").c_str());
  zs::GradPtrs g;
  int rc = gather(c, grads, &g, who);
  if (rc) return rc;
  const int64_t S = c->shard_len;
  float* stage = reinterpret_cast<float*>(c->ws + c->lay.stage_off);
  double* partials = reinterpret_cast<double*>(c->ws + c->lay.partials_off);
  const int32_t n_final = S ? zs::final_partials(S) : 0;
  hipError_t e = hipSuccess;
  if (n_final)
    e = state_dev ? zs::launch_sumsq_f16(c->M, g, S, partials,
                                         reinterpret_cast<const zs::AmpState*>(state_dev),
                                         stage, c->lds.stage_norm, c->max_groups, c->stream)
                  : zs::launch_sumsq(c->M, g, S, partials, stage, c->lds.stage_norm,
                                     c->max_groups, c->stream);
  if (e == hipSuccess)
    e = zs::launch_sumsq_total(partials + zs::level1_partials(S), n_final, sumsq_dev, c->stream);
  return e == hipSuccess ? ZS_OK : zs::ehip(who, e);
}

}  // namespace

extern "C" int zero_offload_grad_sumsq(zs_offload* c, const void* const* grads,
                                       double* sumsq_dev) {
  if (!c) return zs::einval("zero_offload_grad_sumsq: ctx is NULL");
  if (c->fp16) return estate("zero_offload_grad_sumsq: fp16 context: use zero_offload_grad_sumsq_amp");
  return offload_sumsq(c, grads, nullptr, sumsq_dev, "zero_offload_grad_sumsq");
}

extern "C" int zero_offload_step_global_norm(zs_offload* c, const void* const* grads, float lr,
                                             float beta1, float beta2, float eps,
                                             float weight_decay, int64_t step,
                                             float max_grad_norm,
                                             const double* global_sumsq_dev) {
  using zs::einval;
  const char* who = "zero_offload_step_global_norm";
  if (!c) return einval("zero_offload_step_global_norm: ctx is NULL");
  if (c->fp16) return estate("zero_offload_step_global_norm: fp16 context: use the _amp calls");
  int rc = zs::check_hparams(lr, beta1, beta2, eps, weight_decay, step);
  if (rc) return rc;
  if (!(max_grad_norm > 0.0f) || isinf(max_grad_norm))
    return einval("zero_offload_step_global_norm: max_grad_norm must be finite and > 0");
  if (!global_sumsq_dev || !aligned(global_sumsq_dev, 8))
    return einval("zero_offload_step_global_norm: global_sumsq_dev must be an aligned device pointer");
  zs::GradPtrs g;
  if ((rc = gather(c, grads, &g, who))) return rc;
  if (c->shard_len == 0) return ZS_OK;
  const zs::HostConsts k =
      host_consts(zs::step_consts(lr, beta1, beta2, eps, weight_decay, step));
  zs::ClipScalars* sc_dev = reinterpret_cast<zs::ClipScalars*>(c->ws + c->lay.scalars_off);
  const hipError_t e = zs::launch_finalize(nullptr, 0, global_sumsq_dev, max_grad_norm, 1,
                                           (c->flags & ZS_SKIP_NONFINITE) ? 1 : 0, sc_dev,
                                           c->stream);
  if (e != hipSuccess) return zs::ehip("zero_offload_step_global_norm: finalize", e);
  return pipeline(c, &k, false, nullptr, who);
}

extern "C" int zero_offload_grad_sumsq_amp(zs_offload* c, const void* const* grads,
                                           const zs_amp_state* state_dev, double* sumsq_dev) {
  if (!c) return zs::einval("zero_offload_grad_sumsq_amp: ctx is NULL");
  if (!c->fp16)
    return estate("zero_offload_grad_sumsq_amp: needs a context created with ZS_FP16");
  if (!state_dev || !aligned(state_dev, 16))
    return zs::einval(
        "zero_offload_grad_sumsq_amp: state_dev must be a 16-byte-aligned device pointer");
  return offload_sumsq(c, grads, state_dev, sumsq_dev, "zero_offload_grad_sumsq_amp");
}

extern "C" int zero_offload_step_amp_global_norm(zs_offload* c, const void* const* grads,
                                                 float lr, float beta1, float beta2, float eps,
                                                 float weight_decay, float max_grad_norm,
                                                 zs_amp_state* state_dev, float growth_factor,
                                                 float backoff_factor, int32_t growth_interval,
                                                 const double* global_sumsq_dev) {
  const char* who = "zero_offload_step_amp_global_norm";
  if (!c) return zs::einval("zero_offload_step_amp_global_norm: ctx is NULL");
  if (!c->fp16)
    return estate("zero_offload_step_amp_global_norm: needs a context created with ZS_FP16");
  zs::AmpParams p;
  int rc = zs::check_amp_args(who, lr, beta1, beta2, eps, weight_decay, max_grad_norm, state_dev,
                              growth_factor, backoff_factor, growth_interval, &p);
  if (rc) return rc;
  if (!global_sumsq_dev || !aligned(global_sumsq_dev, 8))
    return zs::einval(
        "zero_offload_step_amp_global_norm: global_sumsq_dev must be an aligned device pointer");
  zs::GradPtrs g;
  if ((rc = gather(c, grads, &g, who))) return rc;
  char* block = c->ws + c->lay.scalars_off;
  const hipError_t e = zs::launch_amp_finalize(
      nullptr, 0, global_sumsq_dev, reinterpret_cast<zs::AmpState*>(state_dev), p,
      reinterpret_cast<zs::ClipScalars*>(block), reinterpret_cast<zs::StepConsts*>(block + 64),
      c->stream);
  if (e != hipSuccess) return zs::ehip("zero_offload_step_amp_global_norm: finalize", e);
  return pipeline(c, nullptr, true, nullptr, who);
}

extern "C" int zero_offload_amp_state_init(zs_offload* c, zs_amp_state* state_dev,
                                           float init_scale) {
  if (!c) return zs::einval("zero_offload_amp_state_init: ctx is NULL");
  if (!state_dev || !aligned(state_dev, 16))
    return zs::einval(
        "zero_offload_amp_state_init: state_dev must be a 16-byte-aligned device pointer");
  if (!(init_scale > 0.0f) || isinf(init_scale))
    return zs::einval("zero_offload_amp_state_init: init_scale must be finite and > 0");
  const hipError_t e = zs::launch_amp_state_init(reinterpret_cast<zs::AmpState*>(state_dev),
                                                 init_scale, c->stream);
  return e == hipSuccess ? ZS_OK : zs::ehip("zero_offload_amp_state_init", e);
}

extern "C" int zero_offload_set_stream(zs_offload* c, void* stream) {
  if (!c) return zs::einval("zero_offload_set_stream: ctx is NULL");
  c->stream = static_cast<hipStream_t>(stream);
  return ZS_OK;
}

extern "C" void zero_offload_destroy(zs_offload* c) { delete c; }

extern "C" int zs_host_adamw(const zs_plan* plan, int64_t shard_off, int64_t n,
                             const float* grad_avg, float coef, float* master, float* exp_avg,
                             float* exp_avg_sq, uint16_t* param, float lr, float beta1,
                             float beta2, float eps, float weight_decay, int64_t step,
                             int32_t n_threads, uint32_t flags) {
  using zs::einval;
  if (!plan) return einval("zs_host_adamw: plan is NULL");
  int rc = zs::check_hparams(lr, beta1, beta2, eps, weight_decay, step);
  if (rc) return rc;
  if (shard_off < 0 || n < 0 || shard_off > plan->shard_len || n > plan->shard_len - shard_off)
    return einval("zs_host_adamw: [shard_off, shard_off + n) must lie inside the shard");
  if (!isfinite(coef)) return einval("zs_host_adamw: coef must be finite");
  if (n_threads < 0 || n_threads > 1024)
    return einval("zs_host_adamw: n_threads must lie in [0, 1024]");
  if (n == 0) return ZS_OK;
  if (flags & ~ZS_FP16) return einval("zs_host_adamw: flags may hold only ZS_FP16");
  if (!grad_avg || !master || !exp_avg || !exp_avg_sq || !param)
    return einval("zs_host_adamw: NULL array");
  const zs::HostConsts k =
      host_consts(zs::step_consts(lr, beta1, beta2, eps, weight_decay, step));
  try {
    const std::vector<zs::HostRun> runs = host_runs(plan);
    zs::HostPool pool(n_threads > 0 ? n_threads : zs::default_host_threads());
    zs::host_adamw(pool, runs.data(), (int32_t)runs.size() - 1, shard_off, n, grad_avg, coef,
                   master, exp_avg, exp_avg_sq, param, k, (flags & ZS_FP16) != 0);
  } catch (const std::bad_alloc&) {
    return enomem("zs_host_adamw: out of host memory");
  } catch (const std::system_error&) {
    return enomem("zs_host_adamw: could not start the host threads");
  }
  return ZS_OK;
}
