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

// fp32 -> IEEE binary16, round to nearest even, from the format's definition:
// NaN -> quiet NaN; |x| >= 65520 (halfway above the largest finite 65504, a tie
// that goes to the even neighbour 2^16) -> Inf; normals rebias the exponent
// (127 -> 15) and round 13 mantissa bits away; below 2^-14 the result is
// x * 2^24 rounded to an integer (subnormals, and 2^-14 itself when it rounds
// up), which for a = 1.m * 2^(e-127) is the 24-bit significand shifted right
// by 126 - e; anything below 2^-25 (and 2^-25 itself, a tie to 0) is zero.
inline uint32_t mask_if(bool c) { return 0u - (uint32_t)c; }

// Written with bit masks rather than branches or conditional expressions, so
// the loop vectorizes: the normal and the subnormal result are both computed and
// the range picks one.  Shift counts are clamped to 1..31 so no shift is
// undefined; the lanes that needed the clamp are never selected.
inline uint16_t f32_to_f16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t r = a - 0x38000000u;
  const uint32_t normal = (r + 0x0FFFu + ((r >> 13) & 1u)) >> 13;
  const uint32_t sig = (a & 0x007FFFFFu) | 0x00800000u;
  uint32_t s = 126u - (a >> 23);  // 14..24 for the subnormal range
  s = (s & ~mask_if(s > 31u)) | (31u & mask_if(s > 31u));
  s = s | (uint32_t)(s == 0u);
  const uint32_t q = sig >> s, rem = sig & ((1u << s) - 1u), half = 1u << (s - 1u);
  const uint32_t up = (uint32_t)(rem > half) | ((uint32_t)(rem == half) & q);
  const uint32_t sub = q + (up & 1u);
  // below 2^-25, and 2^-25 itself (a tie to the even 0): zero
  uint32_t h = sub & mask_if(a >= 0x33000000u);
  const uint32_t is_normal = mask_if(a >= 0x38800000u);
  const uint32_t is_inf = mask_if(a >= 0x477FF000u);
  const uint32_t is_nan = mask_if(a > 0x7F800000u);
  h = (h & ~is_normal) | (normal & is_normal);
  h = (h & ~is_inf) | (0x7C00u & is_inf);
  h = (h & ~is_nan) | (0x7E00u & is_nan);
  return (uint16_t)(sign | h);
}

inline uint16_t f32_to_bf16_rne(float x) {  // a NaN stays a quiet NaN
  uint32_t b;
  memcpy(&b, &x, sizeof b);
  const uint32_t rne = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  const uint32_t qnan = (b >> 16) | 0x40u;
  return (uint16_t)(((b & 0x7FFFFFFFu) > 0x7F800000u) ? qnan : rne);
}

template <bool F16>
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
    out[i] = F16 ? f32_to_f16_rne(pn) : f32_to_bf16_rne(pn);
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
                const HostConsts& k, bool out_f16) {
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
      if (out_f16)
        adamw_span<true>(e - s, g + i, coef, p + i, m + i, v + i, out + i, k.beta1, k.beta2,
                         k.c1, k.c2, k.alpha, k.bhat, k.eps, d);
      else
        adamw_span<false>(e - s, g + i, coef, p + i, m + i, v + i, out + i, k.beta1, k.beta2,
                          k.c1, k.c2, k.alpha, k.bhat, k.eps, d);
      s = e;
    }
  });
}

}  // namespace zs
