// internal.h -- types shared by the planner, the kernels and the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace zs {

// A run of the shard with one weight-decay flag (padding joins a neighbouring
// run; it is zero in every array and stays zero under either flag).  The step
// kernel finds the run of each element by binary search over `start`.
struct Run {
  int64_t start;  // shard offset, a multiple of 8 elements
  int32_t flags;  // bit 0: weight decay applies
  int32_t pad;
};
static_assert(sizeof(Run) == 16, "run descriptor is 16 bytes");

struct Segment {
  int64_t shard_off, len, tensor, tensor_off;
  int32_t decay;
};

// A piece of a tensor segment (at most kPieceElems elements) for the state
// export/import kernel: shard offset, offset in the canonical order (tensors
// concatenated without padding), length.
struct Piece {
  int64_t shard_off, canon_off;
  int32_t len, pad;
};
static_assert(sizeof(Piece) == 24, "piece descriptor is 24 bytes");
constexpr int64_t kPieceElems = 65536;

// Per-step constants, each computed in fp64 from the fp32 hyper-parameters
// and rounded once to fp32.
struct StepConsts {
  float beta1, beta2;
  float c1, c2;       // 1 - beta1, 1 - beta2
  float alpha;        // lr / (1 - beta1^t)
  float bhat;         // sqrt(1 - beta2^t)
  float eps;
  float decay_mul;    // 1 - lr * wd (decayed elements; others use 1)
};

constexpr int kMaxM = 16;

// b^t in fp64 by binary powering: square-and-multiply over the bits of t from
// the lowest, each product rounded once -- a fixed sequence of IEEE multiplies,
// so host and device compute the same bits (used for the bias corrections).
__host__ __device__ inline double pow_int(double b, int64_t t) {
  double r = 1.0, x = b;
  while (t > 0) {
    if (t & 1) r = r * x;
    x = x * x;
    t >>= 1;
  }
  return r;
}

struct GradPtrs {
  const uint16_t* p[kMaxM];
};

// Device workspace layout (offsets in bytes from the workspace base).
struct WorkspaceLayout {
  size_t runs_off, runs_bytes;  // n_runs + 1 Run entries (the last is a sentinel)
  size_t pieces_off, pieces_bytes;  // n_pieces Piece entries
  size_t partials_off;          // sumsq_partials(shard_len) doubles
  size_t scalars_off;           // ClipScalars
  size_t total;
};

// Written by the finalize kernel, read by the step kernel.
struct ClipScalars {
  double sumsq;    // sum of g^2 of the reduced gradient
  double norm;     // sqrt(sumsq)
  float coef;      // clip coefficient applied to g (1 when not clipping)
  uint32_t skip;   // nonzero: leave the state untouched this step
  uint32_t pad[2];
};

// fp64 partial sums of the norm pass: level-1 (one per 2048-element tile) followed
// by level-2 (one per 8192 level-1 partials); the finalize step sums the level-2
// ones, final_partials of them starting at level1_partials.
int64_t level1_partials(int64_t shard_len);
int64_t sumsq_partials(int64_t shard_len);
int32_t final_partials(int64_t shard_len);

// Kernel launchers (kernels.hip).  All enqueue on `stream`.
// The norm pass over a non-empty shard: both partial levels into `partials`.
hipError_t launch_sumsq(int M, const GradPtrs& g, int64_t shard_len, double* partials,
                        hipStream_t stream);
// Reduces the partials (or takes *external_sumsq when non-null) into *out.
hipError_t launch_finalize(const double* partials, int32_t n_partials,
                           const double* external_sumsq, float max_norm, int clip,
                           int skip_nonfinite, ClipScalars* out, hipStream_t stream);
hipError_t launch_sumsq_total(const double* partials, int32_t n_partials, double* out,
                              hipStream_t stream);
// waves_per_cu > 0 caps the resident waves per CU of the step kernel (0: no cap).
// Copies fp32 master/m/v between the shard and the canonical order over the
// piece table (export: shard -> canonical; import: canonical -> shard, which
// also writes param = bf16_rne(master) for the imported elements).
hipError_t launch_state_copy(bool do_export, const Piece* pieces, int64_t n_pieces,
                             float* master, float* m, float* v, uint16_t* param, float* c_master,
                             float* c_m, float* c_v, hipStream_t stream);
hipError_t launch_step(int M, bool use_clip, const GradPtrs& g, float* master, float* m,
                       float* v, uint16_t* param, int64_t shard_len, const Run* runs,
                       int32_t n_runs, const ClipScalars* clip, const StepConsts& k,
                       int32_t waves_per_cu, hipStream_t stream);

}  // namespace zs

struct zs_plan {
  int32_t world_size = 1, rank = 0, align = 64;
  int64_t bucket_cap = 0;
  std::vector<int64_t> numel;
  std::vector<uint8_t> decay;
  std::vector<int64_t> tensor_flat_off;
  std::vector<int64_t> tensor_segment;  // segment index of the tensor's piece, or -1
  std::vector<int64_t> bucket_off, bucket_len;
  std::vector<zs::Segment> segments;
  std::vector<zs::Run> runs;
  std::vector<zs::Piece> pieces;
  int64_t shard_len = 0, padded_total = 0, total_params = 0;
};
