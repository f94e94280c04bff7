// host_step.cpp -- the AdamW update on host cores and its thread pool (see host.h).
//
// Built by the host compiler with -O3 -ffp-contract=off: every operation below
// is one IEEE fp32 rounding (x86 vector division and square root are correctly
// rounded), so the update gives the same bits as the device kernels whatever
// vector width the CPU offers.  The inner loop is compiled three times
// (AVX-512, AVX2, baseline SSE2) and the loader picks the widest the CPU runs.
#include "host.h"

#include <sched.h>
#include <string.h>
#include <xmmintrin.h>

#include <algorithm>

namespace zs {

namespace {

// The SSE control word at power-on: all exceptions masked, round to nearest,
// no flush-to-zero, no denormals-are-zero.
constexpr unsigned kDefaultMxcsr = 0x1F80u;

// ZS_HOST_ONE_ISA builds one baseline version instead (for ThreadSanitizer
// builds: the clones' load-time resolver runs before that runtime starts).
#ifdef ZS_HOST_ONE_ISA
#define ZS_ISA_CLONES
#else
#define ZS_ISA_CLONES __attribute__((target_clones("avx512f", "avx2", "default")))
#endif

ZS_ISA_CLONES void adamw_span(
    int64_t n, const float* __restrict g, float coef, float* __restrict p, float* __restrict m,
    float* __restrict v, uint16_t* __restrict out, float beta1, float beta2, float c1, float c2,
    float alpha, float bhat, float eps, float d) {
  for (int64_t i = 0; i < n; i++) {
    const float gq = g[i] * coef;
    const float mN = beta1 * m[i];
    const float mG = c1 * gq;
    const float m1 = mN + mG;
    const float gg = gq * gq;
    const float vN = beta2 * v[i];
    const float vG = c2 * gg;
    const float v1 = vN + vG;
    const float r = __builtin_sqrtf(v1);
    const float q = r / bhat;
    const float den = q + eps;
    const float p1 = p[i] * d;
    const float u = m1 / den;
    const float w = alpha * u;
    const float pn = p1 - w;
    p[i] = pn;
    m[i] = m1;
    v[i] = v1;
    // bf16 round to nearest even; a NaN stays a quiet NaN
    uint32_t b;
    memcpy(&b, &pn, sizeof b);
    const uint32_t rne = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    const uint32_t qnan = (b >> 16) | 0x40u;
    out[i] = (uint16_t)(((b & 0x7FFFFFFFu) > 0x7F800000u) ? qnan : rne);
  }
}

}  // namespace

HostPool::HostPool(int n_threads) : n_(n_threads < 1 ? 1 : n_threads) {
  threads_.reserve((size_t)n_);
  for (int i = 0; i < n_; i++) threads_.emplace_back([this, i] { loop(i); });
}

HostPool::~HostPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  wake_.notify_all();
  for (auto& t : threads_) t.join();
}

void HostPool::loop(int id) {
  _mm_setcsr(kDefaultMxcsr);
  uint64_t seen = 0;
  for (;;) {
    const std::function<void(int, int)>* job;
    {
      std::unique_lock<std::mutex> lk(mu_);
      wake_.wait(lk, [&] { return stop_ || generation_ != seen; });
      if (stop_) return;
      seen = generation_;
      job = job_;
    }
    (*job)(id, n_);
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (--pending_ == 0) done_.notify_one();
    }
  }
}

void HostPool::run(const std::function<void(int, int)>& job) {
  std::unique_lock<std::mutex> lk(mu_);
  job_ = &job;
  pending_ = n_;
  generation_++;
  wake_.notify_all();
  done_.wait(lk, [&] { return pending_ == 0; });
  job_ = nullptr;
}

int default_host_threads() {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  const unsigned h = std::thread::hardware_concurrency();
  return h > 0 ? (int)h : 1;
}

void host_adamw(HostPool& pool, const HostRun* runs, int32_t n_runs, int64_t shard_off, int64_t n,
                const float* g, float coef, float* p, float* m, float* v, uint16_t* out,
                const HostConsts& k) {
  if (n <= 0) return;
  pool.run([&](int id, int nw) {
    // contiguous slices, cut on 64-element (256-byte) boundaries
    const int64_t per = ((n + nw - 1) / nw + 63) / 64 * 64;
    const int64_t lo = std::min(n, per * id), hi = std::min(n, lo + per);
    if (lo >= hi) return;
    const int64_t s_lo = shard_off + lo, s_hi = shard_off + hi;
    // the run holding s_lo: the last run whose start is <= s_lo
    const HostRun* r = std::upper_bound(runs, runs + n_runs, s_lo,
                                        [](int64_t e, const HostRun& x) { return e < x.start; }) -
                       1;
    for (int64_t s = s_lo; s < s_hi; r++) {
      const int64_t e = std::min(s_hi, r[1].start);  // r[1] exists: the table ends with a sentinel
      const float d = (r->flags & 1) ? k.decay_mul : 1.0f;
      const int64_t i = s - shard_off;
      adamw_span(e - s, g + i, coef, p + i, m + i, v + i, out + i, k.beta1, k.beta2, k.c1, k.c2,
                 k.alpha, k.bhat, k.eps, d);
      s = e;
    }
  });
}

}  // namespace zs
