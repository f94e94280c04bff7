// static_step.hip -- zero_shard_step_static: the bf16 shard step for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// zero_shard_step needs a context bound to a caller-allocated workspace (the
// run and tile-flag tables, the norm partials, the clip scalars).  This entry
// point takes the plan instead and keeps that workspace in `scratch`, a
// file-scope device array of kScratchBytes that every GPU the library runs on
// holds until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the first call on
// a device, with that device current, resolves the device address with
// hipGetSymbolAddress and keeps it per device, and every launch and copy uses
// that address.  The kernels are the ones zero_shard_step launches, with the
// same arithmetic, so both entry points give the same bits.
//
// Every call on a GPU shares that GPU's scratch and leaves its contents there:
// each call first writes the plan's tables into it (the run table through
// kernel arguments, the tile flags computed from it on the device, so a call
// enqueues kernels only and can be captured in a graph), and every partial sum
// and scalar a kernel reads is written earlier in the same call, so nothing
// has to start at zero.  Calls that overlap on one GPU (other host threads, other
// streams) race on the scratch; calls ordered on one stream do not.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <string>

#include "../../include/zeroshard.h"
#include "abi_internal.h"
#include "internal.h"
#include "lds.h"

namespace {

constexpr size_t kScratchBytes = ZS_STATIC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch parts are 256-byte aligned");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// What the first call on a device resolved: the scratch's device address and
// the device figures the LDS reservations are checked against.
struct DeviceSetup {
  bool ready = false;
  unsigned char* ptr = nullptr;  // device address of `scratch` on this device
  int32_t n_cu = 256;
  size_t lds_cu = zs::kLdsPerCuDefault, per_wg = 0, static_lds = 0;
};

std::mutex g_setup_mu;
DeviceSetup g_setup[kMaxDevices];

int device_setup(hipStream_t stream, DeviceSetup* out) {
  const char* who = "zero_shard_step_static";
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return zs::ehip(who, e);
  if (dev < 0 || dev >= kMaxDevices)
    return zs::einval("zero_shard_step_static: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_setup_mu);
  DeviceSetup& d = g_setup[dev];
  if (!d.ready) {
    // the set-up queries below are not stream work and would break a capture in
    // progress: refuse before making any of them
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return zs::ehip("zero_shard_step_static: capture status", e);
    if (cs != hipStreamCaptureStatusNone)
      return zs::einval("zero_shard_step_static: the first call on a device must run outside "
                        "graph capture (it resolves the static scratch and queries the device)");
    DeviceSetup n;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return zs::ehip("zero_shard_step_static: scratch address", e);
    n.ptr = static_cast<unsigned char*>(p);
    int cu = 0, per_cu = 0, per_wg = 0;
    e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&per_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return zs::ehip("zero_shard_step_static: device query", e);
    n.n_cu = cu > 0 ? cu : 256;
    n.lds_cu = per_cu > 0 ? (size_t)per_cu : zs::kLdsPerCuDefault;
    n.per_wg = per_wg > 0 ? (size_t)per_wg : zs::kLdsPerWorkgroupFallback;
    for (int M = 1; M <= ZS_MAX_M; M++) {
      size_t s = 0;
      if ((e = zs::reserved_kernels_static_lds(M, &s)) != hipSuccess)
        return zs::ehip("zero_shard_step_static: kernel attributes", e);
      if (s > n.static_lds) n.static_lds = s;
    }
    n.ready = true;
    d = n;
  }
  *out = d;
  return ZS_OK;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Scratch layout of one call: the run table (with its sentinel), the tile
// flags, the norm partials (clipped steps only) and the 256-byte clip scalars.
struct ScratchLayout {
  size_t runs_off, runs_bytes, tflags_off, tflags_bytes, partials_off, scalars_off, total;
};

ScratchLayout scratch_layout(const zs_plan* plan, bool clip) {
  ScratchLayout l;
  l.runs_off = 0;
  l.runs_bytes = plan->run_table.size() * sizeof(zs::Run);
  l.tflags_off = round256(l.runs_bytes);
  l.tflags_bytes = plan->tile_flags.size() * sizeof(uint32_t);
  l.partials_off = l.tflags_off + round256(l.tflags_bytes);
  const size_t partials = clip ? (size_t)zs::sumsq_partials(plan->shard_len) * sizeof(double) : 0;
  l.scalars_off = l.partials_off + round256(partials);
  l.total = l.scalars_off + 256;
  return l;
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int zero_shard_step_static(const zs_plan* plan, int32_t M, void* param_bf16,
                                      float* master, float* exp_avg, float* exp_avg_sq,
                                      const void* const* grads, float lr, float beta1,
                                      float beta2, float eps, float weight_decay, int64_t step,
                                      float max_grad_norm, void* stream) {
  using zs::einval;
  // every argument check comes before the first device call
  if (!plan) return einval("zero_shard_step_static: plan is NULL");
  if (M < 1 || M > ZS_MAX_M) return einval("zero_shard_step_static: M must lie in [1, 16]");
  if (!param_bf16 || !master || !exp_avg || !exp_avg_sq || !grads)
    return einval("zero_shard_step_static: NULL buffer");
  if (!al16(param_bf16) || !al16(master) || !al16(exp_avg) || !al16(exp_avg_sq))
    return einval("zero_shard_step_static: buffers must be 16-byte aligned");
  zs::GradPtrs g{};
  for (int j = 0; j < M; j++) {
    if (!grads[j] || !al16(grads[j]))
      return einval(
          "zero_shard_step_static: every grads[j] must be a non-NULL 16-byte-aligned pointer");
    g.p[j] = static_cast<const uint16_t*>(grads[j]);
  }
  if (int rc = zs::check_hparams(lr, beta1, beta2, eps, weight_decay, step)) return rc;
  if (isnan(max_grad_norm) || isinf(max_grad_norm))
    return einval("zero_shard_step_static: max_grad_norm must be finite");
  if (plan->run_table.size() > 0x3fffffff)
    return einval("zero_shard_step_static: too many weight-decay runs");
  const bool clip = max_grad_norm > 0.0f;
  const ScratchLayout lay = scratch_layout(plan, clip);
  if (lay.total > kScratchBytes)
    return einval(("zero_shard_step_static: this shard needs " + std::to_string(lay.total) +
                   " bytes of scratch (run and tile-flag tables" +
                   std::string(clip ? ", norm partials" : "") + "), more than the " +
                   std::to_string(kScratchBytes) +
                   " the static scratch holds; use zero_shard_init with a workspace")
                      .c_str());
  int32_t override_waves;
  if (!zs::parse_waves_override(getenv("ZS_WAVES_PER_CU"), &override_waves))
    return einval("zero_shard_step_static: ZS_WAVES_PER_CU must be 0 (no cap) or 3..64");
  const int64_t S = plan->shard_len;
  if (S == 0) return ZS_OK;

  hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceSetup d;
  if (int rc = device_setup(st, &d)) return rc;
  const zs::LdsPlan lds = zs::lds_plan(M, S, d.n_cu, d.lds_cu, override_waves);
  if (!zs::lds_plan_fits(lds, d.static_lds, d.per_wg, d.lds_cu))
    return einval("zero_shard_step_static: an LDS reservation exceeds the device's "
                  "per-workgroup limit");

  unsigned char* base = d.ptr;  // the scratch's device address, never the symbol
  const int32_t n_runs = (int32_t)(plan->run_table.size() - 1);
  zs::Run* runs_dev = reinterpret_cast<zs::Run*>(base + lay.runs_off);
  uint32_t* tflags_dev = reinterpret_cast<uint32_t*>(base + lay.tflags_off);
  // the run table travels in kernel arguments; the tile flags are built from it
  // on the device: the call enqueues kernels only
  hipError_t e = zs::launch_store_words(reinterpret_cast<const uint32_t*>(plan->run_table.data()),
                                        (int64_t)(lay.runs_bytes / sizeof(uint32_t)),
                                        reinterpret_cast<uint32_t*>(runs_dev), st);
  if (e == hipSuccess && lay.tflags_bytes)
    e = zs::launch_tile_flags(runs_dev, n_runs, S, tflags_dev, st);
  if (e != hipSuccess) return zs::ehip("zero_shard_step_static: table upload", e);
  zs::RunTable rt;
  rt.runs = runs_dev;
  rt.tile_flags = lay.tflags_bytes ? tflags_dev : nullptr;
  rt.n_runs = n_runs;
  zs::ClipScalars* sc = reinterpret_cast<zs::ClipScalars*>(base + lay.scalars_off);
  const int64_t max_groups = zs::max_groups_from_env();
  if (clip) {
    double* partials = reinterpret_cast<double*>(base + lay.partials_off);
    e = zs::launch_sumsq(M, g, S, partials, nullptr, 0, max_groups, st);
    if (e != hipSuccess) return zs::ehip("zero_shard_step_static: norm pass", e);
    e = zs::launch_finalize(partials + zs::level1_partials(S), zs::final_partials(S), nullptr,
                            max_grad_norm, 1, 0, sc, st);
    if (e != hipSuccess) return zs::ehip("zero_shard_step_static: norm finalize", e);
  }
  const zs::StepConsts k = zs::step_consts(lr, beta1, beta2, eps, weight_decay, step);
  e = zs::launch_step(M, clip, g, master, exp_avg, exp_avg_sq, static_cast<uint16_t*>(param_bf16),
                      S, rt, sc, k, lds.step, max_groups, st);
  if (e != hipSuccess) return zs::ehip("zero_shard_step_static: step kernel", e);
  return ZS_OK;
}
