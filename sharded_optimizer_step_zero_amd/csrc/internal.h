// internal.h -- types shared by the planner, the kernels and the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace zs {

// A run of the shard with one weight-decay flag (padding joins a neighbouring
// run; it is zero in every array and stays zero under either flag).  The step
// kernels take a tile's flag from the tile-flag table (RunTable) and search the
// runs by `start` only inside tiles that straddle a boundary.
struct Run {
  int64_t start;  // shard offset, a multiple of 8 elements
  int32_t flags;  // bit 0: weight decay applies
  int32_t pad;
};
static_assert(sizeof(Run) == 16, "run descriptor is 16 bytes");

// Elements per step-kernel tile (one single-wave workgroup each).
constexpr int64_t kStepTileElems = 256;

// The decay runs as the step kernels read them: the run table (n_runs entries
// and a sentinel) and, when n_runs > 1, 2 bits per tile, 16 tiles per word:
// bit 0 is the decay flag of a tile inside one run, bit 1 marks a tile that
// straddles a run boundary (its lanes then look the run up themselves).
struct RunTable {
  const Run* runs;
  const uint32_t* tile_flags;  // null when n_runs == 1
  int32_t n_runs;
};

// Words of the tile-flag table of a shard (0 when there is one run).
inline int64_t tile_flag_words(int64_t shard_len, int64_t n_runs) {
  if (n_runs <= 1) return 0;
  const int64_t tiles = (shard_len + kStepTileElems - 1) / kStepTileElems;
  return (tiles + 15) / 16;
}

struct Segment {
  int64_t shard_off, len, tensor, tensor_off;
  int32_t decay;
};

// A piece of a tensor segment for the state export/import kernel: shard
// offset, offset in the canonical order (tensors concatenated without
// padding), length.  A plan's piece table holds its whole pieces (kPieceElems
// elements, copied as kPieceElems / kCopyPart parts) first, then the
// remainder of every segment as parts of at most kCopyPart elements.
struct Piece {
  int64_t shard_off, canon_off;
  int32_t len, pad;
};
static_assert(sizeof(Piece) == 24, "piece descriptor is 24 bytes");
constexpr int64_t kPieceElems = 65536;
constexpr int64_t kCopyPart = 256;  // elements per work-group of the copy kernel

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

// Device workspace layout (offsets in bytes from the workspace base, in this
// order, each part 256-byte aligned).
struct WorkspaceLayout {
  size_t stage_off, stage_bytes;  // shard_len floats with ZS_STAGE_AVERAGE, else empty
  size_t runs_off, runs_bytes;  // n_runs + 1 Run entries (the last is a sentinel)
  size_t tflags_off, tflags_bytes;  // tile_flag_words(shard_len, n_runs) words
  size_t pieces_off, pieces_bytes;  // n_pieces Piece entries
  size_t partials_off;          // sumsq_partials(shard_len) doubles
  size_t scalars_off;           // 256-byte block: ClipScalars, then StepConsts at +64
  size_t total;
};

// Written by the finalize kernel, read by the step kernel.
struct ClipScalars {
  double sumsq;     // sum of g^2 of the reduced (and unscaled) gradient
  double norm;      // sqrt(sumsq)
  float coef;       // clip coefficient applied to g (1 when not clipping)
  uint32_t skip;    // nonzero: leave the state untouched this step
  float inv_scale;  // loss-scaled path: fp32(1/scale) of the scale the grads carry
  uint32_t pad;
};

// Device state of the dynamic loss scaler (layout of zs_amp_state).
struct AmpState {
  float scale;
  int32_t growth_tracker;
  int64_t applied_steps;
};
static_assert(sizeof(AmpState) == 16, "loss-scaler state is 16 bytes");

struct AmpParams {
  float lr, beta1, beta2, eps, weight_decay, max_norm, growth, backoff;
  int32_t interval, clip;
};

// Per-step constants, each computed in fp64 from the fp32 hyper-parameters and
// rounded once to fp32 (host for the plain step, device for the loss-scaled
// step, whose step count lives on the device).
__host__ __device__ inline StepConsts step_consts(float lr, float beta1, float beta2, float eps,
                                                  float wd, int64_t t) {
  const double b1 = beta1, b2 = beta2, l = lr;
  const double bc1 = 1.0 - pow_int(b1, t);
  const double bc2 = 1.0 - pow_int(b2, t);
  StepConsts k;
  k.beta1 = beta1;
  k.beta2 = beta2;
  k.c1 = (float)(1.0 - b1);
  k.c2 = (float)(1.0 - b2);
  k.alpha = (float)(l / bc1);
  k.bhat = (float)__builtin_sqrt(bc2);
  k.eps = eps;
  k.decay_mul = (float)(1.0 - l * (double)wd);
  return k;
}

// fp64 partial sums of the norm pass: level-1 (one per 2048-element tile) followed
// by level-2 (one per 8192 level-1 partials); the finalize step sums the level-2
// ones, final_partials of them starting at level1_partials.
int64_t level1_partials(int64_t shard_len);
int64_t sumsq_partials(int64_t shard_len);
int32_t final_partials(int64_t shard_len);

// ZS_MAX_GROUPS_PER_LAUNCH from the environment (0 when unset or invalid).
int64_t max_groups_from_env();

// Kernel launchers (kernels.hip).  All enqueue on `stream`.  A grid beyond what
// one dispatch carries (2^32 - 1 work-items) goes out as consecutive slices;
// max_groups > 0 caps the work-groups of each slice below that (a context takes
// it from ZS_MAX_GROUPS_PER_LAUNCH at init; 0 leaves only the dispatch limit).
// lds / stage_lds: the dynamic LDS each work-group of a capped launch reserves
// (lds.h; checked against the device's limits when the context is made).
//
// The norm pass over a non-empty shard: both partial levels into `partials`.
// stage (nullable): also store the fp32 averages, shard_len floats, for
// launch_step_staged.
hipError_t launch_sumsq(int M, const GradPtrs& g, int64_t shard_len, double* partials,
                        float* stage, size_t stage_lds, int64_t max_groups, hipStream_t stream);
// Reduces the partials (or takes *external_sumsq when non-null) into *out.
hipError_t launch_finalize(const double* partials, int32_t n_partials,
                           const double* external_sumsq, float max_norm, int clip,
                           int skip_nonfinite, ClipScalars* out, hipStream_t stream);
hipError_t launch_sumsq_total(const double* partials, int32_t n_partials, double* out,
                              hipStream_t stream);
// Loss-scaled (fp16) path: the norm pass on the unscaled average, the finalize
// step that also computes the step constants on the device and updates the
// scaler, the step kernel, and the scaler initialisation.
hipError_t launch_sumsq_f16(int M, const GradPtrs& g, int64_t shard_len, double* partials,
                            const AmpState* st, float* stage, size_t stage_lds,
                            int64_t max_groups, hipStream_t stream);
// external (nullable): a global sum of squares used instead of the partials.
hipError_t launch_amp_finalize(const double* partials, int32_t n_partials,
                               const double* external, AmpState* st, const AmpParams& p,
                               ClipScalars* out, StepConsts* kout, hipStream_t stream);
hipError_t launch_step_f16(int M, const GradPtrs& g, float* master, float* m, float* v,
                           uint16_t* param, int64_t shard_len, const RunTable& rt,
                           const ClipScalars* clip, const StepConsts* k, size_t lds,
                           int64_t max_groups, hipStream_t stream);
hipError_t launch_amp_state_init(AmpState* st, float scale, hipStream_t stream);
// The step on the averages a norm pass staged (amp: constants *kd and an fp16
// param; otherwise kh and a bf16 param).
hipError_t launch_step_staged(bool amp, const float* stage, float* master, float* m, float* v,
                              uint16_t* param, int64_t shard_len, const RunTable& rt,
                              const ClipScalars* clip, const StepConsts& kh, const StepConsts* kd,
                              size_t lds, int64_t max_groups, hipStream_t stream);

// Copies fp32 master/m/v between the shard and the canonical order over the
// piece table (export: shard -> canonical; import: canonical -> shard, which
// also writes param = bf16_rne(master), or fp16 when param_f16, for the
// imported elements).
hipError_t launch_state_copy(bool do_export, bool param_f16, const Piece* pieces,
                             int64_t n_pieces, int64_t n_whole, float* master, float* m,
                             float* v, uint16_t* param, float* c_master, float* c_m, float* c_v,
                             size_t lds, int64_t max_groups, hipStream_t stream);
// The fused bf16 step (use_clip: scale by the coefficient in *clip, or skip).
hipError_t launch_step(int M, bool use_clip, const GradPtrs& g, float* master, float* m,
                       float* v, uint16_t* param, int64_t shard_len, const RunTable& rt,
                       const ClipScalars* clip, const StepConsts& k, size_t lds,
                       int64_t max_groups, hipStream_t stream);

// n_words 32-bit words from host memory to device memory through kernel
// arguments (launches of at most 512 words; the host data is read before the
// call returns).  No copy engine, no allocation: capturable in a graph.
hipError_t launch_store_words(const uint32_t* host_words, int64_t n_words, uint32_t* dst,
                              hipStream_t stream);
// The tile-flag table (tile_flag_words(shard_len, n_runs) words) from a device
// run table with its sentinel, as the planner computes it on the host.
hipError_t launch_tile_flags(const Run* runs, int32_t n_runs, int64_t shard_len, uint32_t* flags,
                             hipStream_t stream);

// The largest static LDS of the kernels that launch with a reservation, for M
// contributions (hipFuncGetAttributes on the current device).
hipError_t reserved_kernels_static_lds(int M, size_t* worst);

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
  std::vector<zs::Run> run_table;     // runs (at least one) + a sentinel at shard_len
  std::vector<uint32_t> tile_flags;   // 2 bits per step tile; empty with one run
  std::vector<zs::Piece> pieces;  // whole pieces first (n_whole_pieces), then parts
  int64_t n_whole_pieces = 0;
  int64_t shard_len = 0, padded_total = 0, total_params = 0;
};
