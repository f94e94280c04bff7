// host.h -- the optimizer step on host cores (the offloaded update) and the
// thread pool that runs it.  Plain C++17, no HIP: host_step.cpp is built by the
// host compiler.
//
// Offloading the optimizer to the host: the shard's fp32 master/m/v stay in
// host memory and the host cores run the Adam step; only the averaged gradient
// goes down and the 16-bit params come back over PCIe (大模型基础设施工程 06:
// §3.3 and §9.3 on ZeRO-Offload, the optimizer offload with pinned memory in
// the DeepSpeed configuration of §11.3, and FAQ Q5 on its throughput).
#pragma once

#include <stdint.h>

#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace zs {

// Same layout as Run: a shard range [start, next start) with one decay flag.
struct HostRun {
  int64_t start;
  int32_t flags;  // bit 0: weight decay applies
  int32_t pad;
};

// Same values as StepConsts (each computed in fp64 and rounded once to fp32).
struct HostConsts {
  float beta1, beta2, c1, c2, alpha, bhat, eps, decay_mul;
};

// A fixed set of worker threads.  run() hands every worker the same job
// (worker index, worker count) and returns when all have finished.  Workers
// start with the default SSE control word (round to nearest, no flush of
// subnormals), whatever the creating thread uses.
class HostPool {
 public:
  explicit HostPool(int n_threads);
  ~HostPool();
  HostPool(const HostPool&) = delete;
  HostPool& operator=(const HostPool&) = delete;
  int size() const { return n_; }
  void run(const std::function<void(int, int)>& job);

 private:
  void loop(int id);
  const int n_;
  std::vector<std::thread> threads_;
  std::mutex mu_;
  std::condition_variable wake_, done_;
  const std::function<void(int, int)>* job_ = nullptr;
  uint64_t generation_ = 0;
  int pending_ = 0;
  bool stop_ = false;
};

// Threads this process may run on (the affinity mask), at least 1.
int default_host_threads();

// AdamW on shard elements [shard_off, shard_off + n): g, p, m, v, out point at
// the first of those n elements.  runs: the plan's run table followed by a
// sentinel whose start is the shard length.  Per element, in this order, each
// step one IEEE fp32 rounding:
//   g' = g * coef; m' = beta1*m + c1*g'; v' = beta2*v + c2*(g'*g');
//   den = sqrt(v')/bhat + eps; p' = p*d - alpha*(m'/den); out = bf16_rne(p')
// with d = decay_mul on decayed runs and 1 elsewhere; out is fp16_rne(p') when
// out_f16 (the loss-scaled path's param copy).
void host_adamw(HostPool& pool, const HostRun* runs, int32_t n_runs, int64_t shard_off, int64_t n,
                const float* g, float coef, float* p, float* m, float* v, uint16_t* out,
                const HostConsts& k, bool out_f16 = false);

}  // namespace zs
