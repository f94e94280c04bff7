// host_step_check.cpp -- the host update and its thread pool (host_step.cpp)
// under sanitizers: AddressSanitizer + UndefinedBehaviorSanitizer for bounds
// and undefined behaviour, ThreadSanitizer for races in the pool's hand-off.
// The same update (bf16 and fp16 param out; masters include values across the
// fp16 range) over a many-run table is run with 1..16 threads, repeatedly
// and from pools created and destroyed in a loop; every result must equal the
// one-thread result bit for bit.  Exit status 0 when all agree.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../sharded_optimizer_step_zero_amd/csrc/host.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float uniform_pm1() {  // inputs only
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((int32_t)(rng >> 32)) * (1.0f / 2147483648.0f);
}

int main() {
  const int64_t S = 300007 * 8;  // a multiple of 8, not of 64
  std::vector<zs::HostRun> runs;
  for (int64_t s = 0; s < S;) {  // runs of uneven lengths, alternating decay
    runs.push_back({s, (int32_t)(runs.size() & 1), 0});
    s += 8 * (1 + (int64_t)((uint32_t)(uniform_pm1() * 1e6f + 1e6f) % 5000));
  }
  runs.push_back({S, 0, 0});
  const int32_t n_runs = (int32_t)runs.size() - 1;
  std::vector<float> g(S), p0(S);
  for (int64_t i = 0; i < S; i++) {
    g[i] = 1e-3f * uniform_pm1();
    // masters over many magnitudes: fp16 subnormals, normals, overflow
    const int k = (int)(i % 7);
    p0[i] = uniform_pm1() * (k == 0 ? 1e-6f : k == 1 ? 3e-5f : k == 2 ? 7e4f : 0.02f);
  }
  const zs::HostConsts k = {0.9f, 0.95f, 0.1f, 0.05f, 1e-3f, 0.2236068f, 1e-8f, 0.9999f};
  for (int f16 = 0; f16 < 2; f16++) {
  std::vector<float> rp, rm, rv;
  std::vector<uint16_t> rb;
  for (int threads : {1, 2, 3, 7, 16}) {
    for (int rep = 0; rep < 3; rep++) {
      zs::HostPool pool(threads);
      std::vector<float> p(p0), m(S, 0.0f), v(S, 0.0f);
      std::vector<uint16_t> b(S, 0);
      // three steps over uneven chunks, the last chunk ragged
      for (int step = 0; step < 3; step++) {
        for (int64_t off = 0; off < S; off += 100000) {
          const int64_t n = off + 100000 <= S ? 100000 : S - off;
          zs::host_adamw(pool, runs.data(), n_runs, off, n, g.data() + off, 0.5f, p.data() + off,
                         m.data() + off, v.data() + off, b.data() + off, k, f16 != 0);
        }
      }
      if (rp.empty()) {
        rp = p, rm = m, rv = v, rb = b;
      } else if (memcmp(rp.data(), p.data(), S * 4) || memcmp(rm.data(), m.data(), S * 4) ||
                 memcmp(rv.data(), v.data(), S * 4) || memcmp(rb.data(), b.data(), S * 2)) {
        fprintf(stderr, "f16=%d threads=%d rep=%d: result differs from one thread\n", f16,
                threads, rep);
        return 1;
      }
    }
  }
  }
  printf("host step check ok: %d runs, 1..16 threads, pools rebuilt, results identical\n", n_runs);
  return 0;
}
