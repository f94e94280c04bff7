// kernels.hip -- the fused ZeRO shard step for gfx950 (MI355X).
//
// The step is one streaming pass over HBM: per element it reads M bf16
// gradient contributions and the fp32 master, m, v (2M + 12 bytes) and writes
// master, m, v and the bf16 param (14 bytes).  At well under one flop per byte
// it is bound by HBM bandwidth, far from the VALU and MFMA limits, so there is
// no matrix-core work here; every element is read and written exactly once.
//
// Launch shape (measured on MI355X): the flat shard is cut into tiles of 256
// elements, one tile per single-wave workgroup, each lane owning 4 consecutive
// elements (one 8-byte load per bf16 stream, one 16-byte load per fp32
// stream; loads and stores non-temporal).  Small, short-lived workgroups
// dispatched in order keep the waves in flight on a compact window of every
// stream, and a cap of a few waves per CU (set through an LDS reservation the
// kernel never touches) keeps the outstanding requests near what HBM serves
// best; both beat a persistent grid-stride loop, which spreads concurrent
// accesses over the whole array.  The tile's weight-decay flag is one
// wave-uniform load from a 2-bit-per-tile table, issued after the vector loads
// so it overlaps their latency; only a tile that straddles a run boundary
// looks its runs up per lane.
//
// Variants on the same design: the loss-scaled fp16 step (fp16 loads, unscale,
// device-side skip and step constants, fp16 re-cast) and the staged step that
// reads the fp32 average a norm pass stored instead of the M contributions.
//
// Arithmetic per element (each operation one fp32 rounding, the build uses
// -ffp-contract=off and correctly rounded division and square root):
//   s = grad_0 + grad_1 + ... + grad_{M-1}  (bf16 widened exactly, in order)
//   g = s / M                               [ * coef when clipping ]
//   m' = beta1*m + c1*g,  v' = beta2*v + c2*(g*g)
//   den = sqrt(v') / bhat + eps
//   p' = p*d - alpha*(m'/den),  param = bf16_rne(p')
// The gradient-accumulation average is the g = (1/M) sum_j grad_j equation of
// Lecture04 notes ("单卡 baseline 与 gradient accumulation 的隐藏假设"); the
// update is AdamW with m and v following the Adam recursion (Lecture04 notes,
// "ZeRO-1"); fp32 accumulation and update as 大模型基础设施工程 06 §9.1
// prescribes.
//
// The optional clip needs the global norm before any update, so it is a
// separate read pass: sumsq_kernel recomputes g over 2048-element tiles and
// accumulates g^2 in fp64 per lane, each workgroup sums in a fixed order,
// sum_blocks_kernel adds fixed blocks of those partials, and finalize_kernel
// adds the remaining few thousand in index order -- run-to-run deterministic.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds.h"

namespace zs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 wave64s per workgroup (norm pass)
constexpr int kVec = 8;        // elements per lane in the norm pass (two groups of 4)
constexpr int64_t kNormTile = (int64_t)kThreads * kVec;
constexpr int64_t kLevel2 = 8192;  // level-1 partials summed by one level-2 workgroup

// Streaming (non-temporal) load: the data is used once, so it should not
// displace anything in L2 or the Infinity Cache.  Measured on MI355X it raises
// the step kernel's bandwidth by about 10% over plain loads.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN is kept as a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}

// fp16 <-> fp32 with the hardware's IEEE conversions: exact widening; narrowing
// rounds to nearest even with overflow to Inf.
__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}
__device__ __forceinline__ uint32_t f2h(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ void adamw(float g, float& p, float& m, float& v, const StepConsts& k,
                                      float d) {
  const float mN = k.beta1 * m;
  const float mG = k.c1 * g;
  const float m1 = mN + mG;
  const float gg = g * g;
  const float vN = k.beta2 * v;
  const float vG = k.c2 * gg;
  const float v1 = vN + vG;
  const float r = __builtin_sqrtf(v1);
  const float q = r / k.bhat;
  const float den = q + k.eps;
  const float p1 = p * d;
  const float u = m1 / den;
  const float w = k.alpha * u;
  p = p1 - w;
  m = m1;
  v = v1;
}

// Index of the run containing shard offset e (runs[0].start == 0 <= e).
__device__ __forceinline__ int32_t find_run(const Run* __restrict__ runs, int32_t n_runs, int64_t e) {
  int32_t lo = 0, hi = n_runs - 1;  // invariant: runs[lo].start <= e, answer in [lo, hi]
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (runs[mid].start <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Decay flag (0 or 1) of element e of tile `tile`, which starts at element
// tile0.  One uniform load of the tile's 2 bits; only a tile that straddles a
// run boundary looks the run up per lane, from a uniform binary search for the
// tile's first run (runs[n_runs] is a sentinel past the shard).
__device__ __forceinline__ uint32_t decay_flag(const RunTable& rt, int64_t tile, int64_t tile0,
                                               int64_t e) {
  if (rt.n_runs == 1) return (uint32_t)rt.runs[0].flags & 1u;
  const uint32_t f = (rt.tile_flags[tile >> 4] >> ((uint32_t)(tile & 15) * 2u)) & 3u;
  if (!(f & 2u)) return f;
  int32_t r = find_run(rt.runs, rt.n_runs, tile0);
  while (rt.runs[r + 1].start <= e) r++;
  return (uint32_t)rt.runs[r].flags & 1u;
}

constexpr int kStepLanes = 64;   // one wave64 per workgroup
constexpr int kStepVec = 4;      // elements per lane
constexpr int kTile = kStepLanes * kStepVec;
static_assert(kTile == kStepTileElems, "tile-flag table and step tiles agree");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streamed outputs are written with buffer stores whose cache policy is
// non-temporal at device scope (LLVM's cache-policy bits NT = 2 | SC1 = 16).
// Measured on MI355X against plain non-temporal stores, same buffers: +1.5% on
// the GPT-1.3B shard, +1.8% on the stress workload, +0.6% on Llama-6.7B; the
// same policy on loads changed nothing.  The resource covers `bytes` from
// `base` (a whole tile; lanes past the shard's end return before storing).
constexpr int kStorePolicy = 2 | 16;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(T* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ void st_out(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, byte_off, 0,
                                         kStorePolicy);
}
__device__ __forceinline__ void st_out(__amdgpu_buffer_rsrc_t r, int byte_off, u32x2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(x, r, byte_off, 0, kStorePolicy);
}

// The four outputs of one lane of a step tile: master, m, v (fp32) and the
// 16-bit param copy, elements [tile0 + 4*lane, tile0 + 4*lane + 4).
__device__ __forceinline__ void store_step(float* master, float* mom1, float* mom2,
                                           uint16_t* param, int64_t tile0, f32x4 p4, f32x4 m4,
                                           f32x4 v4, u32x2 pk) {
  const int lane = threadIdx.x;
  st_out(out_rsrc(master + tile0, kTile * 4), lane * 16, p4);
  st_out(out_rsrc(mom1 + tile0, kTile * 4), lane * 16, m4);
  st_out(out_rsrc(mom2 + tile0, kTile * 4), lane * 16, v4);
  st_out(out_rsrc(param + tile0, kTile * 2), lane * 8, pk);
}

template <int M, bool CLIP>
__global__ __launch_bounds__(kStepLanes) void step_kernel(
    GradPtrs g, float* __restrict__ master, float* __restrict__ mom1, float* __restrict__ mom2,
    uint16_t* __restrict__ param, int64_t n, RunTable rt, const ClipScalars* __restrict__ clip,
    StepConsts k, int64_t group0) {
  const int64_t tile = group0 + blockIdx.x;
  const int64_t tile0 = tile * kTile;
  const int64_t e = tile0 + (int64_t)threadIdx.x * kStepVec;
  if (e >= n) return;  // n is a multiple of 8: a lane's 4 elements are all in or all out

  // vector loads first: the M contributions, then master, m, v -- all
  // non-temporal, since every byte is touched once per step
  u32x2 w[M];
#pragma unroll
  for (int j = 0; j < M; j++) w[j] = ld_stream(reinterpret_cast<const u32x2*>(g.p[j] + e));
  f32x4 p4 = ld_stream(reinterpret_cast<const f32x4*>(master + e));
  f32x4 m4 = ld_stream(reinterpret_cast<const f32x4*>(mom1 + e));
  f32x4 v4 = ld_stream(reinterpret_cast<const f32x4*>(mom2 + e));

  // the tile's decay flag, issued after the vector loads
  const float d = decay_flag(rt, tile, tile0, e) ? k.decay_mul : 1.0f;
  float coef = 1.0f;
  if (CLIP) {
    if (clip->skip) return;  // uniform: the whole grid leaves the state untouched
    coef = clip->coef;
  }

  float s[kStepVec];
  s[0] = bf16_lo(w[0].x); s[1] = bf16_hi(w[0].x);
  s[2] = bf16_lo(w[0].y); s[3] = bf16_hi(w[0].y);
#pragma unroll
  for (int j = 1; j < M; j++) {
    s[0] = s[0] + bf16_lo(w[j].x); s[1] = s[1] + bf16_hi(w[j].x);
    s[2] = s[2] + bf16_lo(w[j].y); s[3] = s[3] + bf16_hi(w[j].y);
  }
  uint32_t b[kStepVec];
#pragma unroll
  for (int q = 0; q < kStepVec; q++) {
    float gq = s[q] / (float)M;
    if (CLIP) gq = gq * coef;
    float p = p4[q], m = m4[q], v = v4[q];
    adamw(gq, p, m, v, k, d);
    p4[q] = p;
    m4[q] = m;
    v4[q] = v;
    b[q] = to_bf16(p);
  }
  u32x2 pb;
  pb.x = b[0] | (b[1] << 16);
  pb.y = b[2] | (b[3] << 16);
  store_step(master, mom1, mom2, param, tile0, p4, m4, v4, pb);
}

// Sum over the workgroup in a fixed order: butterfly inside each wave64, then
// the four wave totals in wave order.  The result is valid in thread 0.
__device__ __forceinline__ double block_sum(double x) {
  __shared__ double wave_tot[kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = x + __shfl_xor(x, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wave_tot[wave] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    t = wave_tot[0];
    for (int w = 1; w < kThreads / 64; w++) t = t + wave_tot[w];
  }
  return t;
}

// Norm pass, level 1: one 2048-element tile per workgroup (in-order, short-lived
// workgroups stream best).  Lane t takes elements [4t, 4t+4) and [1024+4t,
// 1024+4t+4) of the tile, so each load and store instruction of the wave covers
// one contiguous stretch (8-byte loads of 16-bit values, 16-byte stores of fp32;
// measured 3.5-4% faster than 8 consecutive elements per lane).  It squares its
// 8 averaged values in fp64 (the square of an fp32 value is exact in fp64), in
// that order, and the workgroup sums in a fixed order.  With STAGE it also
// stores the averages for the staged step.
template <int M, bool STAGE>
__global__ __launch_bounds__(kThreads) void sumsq_kernel(GradPtrs g, int64_t n,
                                                         double* __restrict__ partials,
                                                         float* __restrict__ stage,
                                                         int64_t group0) {
  const int64_t blk = group0 + blockIdx.x;
  const int64_t base = blk * kNormTile + (int64_t)threadIdx.x * 4;
  // every load of both halves first: a staged store must not hold the second
  // half's loads back (the compiler cannot tell stage from the contributions)
  bool in[2];
  u32x2 w[2][M];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int64_t e = base + h * (kNormTile / 2);
    in[h] = e < n;  // n is a multiple of 8: 4-element groups are all in or all out
    if (in[h]) {
#pragma unroll
      for (int j = 0; j < M; j++) w[h][j] = ld_stream(reinterpret_cast<const u32x2*>(g.p[j] + e));
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    if (!in[h]) continue;
    float s[4];
    s[0] = bf16_lo(w[h][0].x); s[1] = bf16_hi(w[h][0].x);
    s[2] = bf16_lo(w[h][0].y); s[3] = bf16_hi(w[h][0].y);
#pragma unroll
    for (int j = 1; j < M; j++) {
      s[0] = s[0] + bf16_lo(w[h][j].x); s[1] = s[1] + bf16_hi(w[h][j].x);
      s[2] = s[2] + bf16_lo(w[h][j].y); s[3] = s[3] + bf16_hi(w[h][j].y);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      s[q] = s[q] / (float)M;
      const double x = (double)s[q];
      acc = acc + x * x;
    }
    if (STAGE) {
      f32x4 a;
      a[0] = s[0]; a[1] = s[1]; a[2] = s[2]; a[3] = s[3];
      st_out(out_rsrc(stage + blk * kNormTile + h * (kNormTile / 2),
                      (int)(kNormTile / 2) * 4),
             threadIdx.x * 16, a);
    }
  }
  const double t = block_sum(acc);
  if (threadIdx.x == 0) partials[blk] = t;
}

// Norm pass, level 2: workgroup b sums partials [b*kLevel2, (b+1)*kLevel2) in a
// fixed order (lane t takes t, t+256, ...; then the fixed workgroup sum).
__global__ __launch_bounds__(kThreads) void sum_blocks_kernel(const double* __restrict__ in,
                                                              int64_t n, double* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kLevel2;
  const int64_t end = base + kLevel2 < n ? base + kLevel2 : n;
  double acc = 0.0;
  for (int64_t i = base + threadIdx.x; i < end; i += kThreads) acc = acc + in[i];
  const double t = block_sum(acc);
  if (threadIdx.x == 0) out[blockIdx.x] = t;
}

__device__ __forceinline__ double sum_partials(const double* __restrict__ partials, int32_t n) {
  double acc = 0.0;
  for (int32_t i = threadIdx.x; i < n; i += kThreads) acc = acc + partials[i];
  return block_sum(acc);
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(
    const double* __restrict__ partials, int32_t n, const double* __restrict__ external,
    float max_norm, int clip, int skip_nonfinite, ClipScalars* __restrict__ out) {
  const double part = external ? 0.0 : sum_partials(partials, n);
  if (threadIdx.x != 0) return;
  const double total = external ? *external : part;
  const double norm = __builtin_sqrt(total);
  float coef = 1.0f;
  if (clip) {
    double c = (double)max_norm / (norm + 1e-6);
    if (c > 1.0) c = 1.0;
    coef = (float)c;
  }
  ClipScalars r;
  r.sumsq = total;
  r.norm = norm;
  r.coef = coef;
  r.skip = (skip_nonfinite && !__builtin_isfinite(total)) ? 1u : 0u;
  r.inv_scale = 1.0f;
  r.pad = 0;
  *out = r;
}

__global__ __launch_bounds__(kThreads) void sumsq_total_kernel(const double* __restrict__ partials,
                                                               int32_t n, double* __restrict__ out) {
  const double t = sum_partials(partials, n);
  if (threadIdx.x == 0) *out = t;
}

// State export/import: one single-wave workgroup per part of at most 256
// elements, the same shape as the step's tiles.  The piece table lists whole
// pieces first (kCopySplit parts each, found by division) and then every other
// part as its own entry, so no workgroup is empty.  A part whose six (seven on
// import) addresses are all 16-byte aligned -- every part when tensor sizes
// are multiples of 4 -- moves 4 elements per lane with 16-byte accesses; any
// other part takes the 4-byte path (still coalesced, 256 B per wave), and a
// 16-byte part's last len % 4 elements are copied one per lane.  The choice is
// per part, so uniform over the workgroup.  Resident waves per CU are capped at kCopyWavesPerCu through an
// LDS reservation, as for the step.  Measured on MI355X against 256-lane
// workgroups over 1,024-element parts and no cap (GPT-1.3B shard, same
// buffers): export 6.81 against 5.70 TB/s, import 6.74 against 5.72; caps 9-14
// swept, 10 best.  On the stress layout (10k tensors, mostly unaligned
// canonical offsets, so mostly the 4-byte path): export 4.72 against 4.59,
// import 5.11 against 5.06.
constexpr int kCopyLanes = 64;
constexpr int32_t kCopySplit = (int32_t)(kPieceElems / kCopyPart);
static_assert(kCopyPart == kCopyLanes * 4, "one 4-element group per lane");

template <bool EXPORT, bool F16>
__device__ __forceinline__ void copy_one(int64_t s, int64_t c, float* __restrict__ master,
                                         float* __restrict__ mom1, float* __restrict__ mom2,
                                         uint16_t* __restrict__ param, float* __restrict__ c_master,
                                         float* __restrict__ c_m, float* __restrict__ c_v) {
  if (EXPORT) {
    c_master[c] = master[s];
    c_m[c] = mom1[s];
    c_v[c] = mom2[s];
  } else {
    const float p = c_master[c];
    master[s] = p;
    mom1[s] = c_m[c];
    mom2[s] = c_v[c];
    param[s] = (uint16_t)(F16 ? f2h(p) : to_bf16(p));
  }
}

__device__ __forceinline__ bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <bool EXPORT, bool F16>
__global__ __launch_bounds__(kCopyLanes) void state_copy_kernel(
    const Piece* __restrict__ pieces, int64_t n_whole, float* __restrict__ master,
    float* __restrict__ mom1, float* __restrict__ mom2, uint16_t* __restrict__ param,
    float* __restrict__ c_master, float* __restrict__ c_m, float* __restrict__ c_v,
    int64_t group0) {
  const int64_t grp = group0 + blockIdx.x;
  const int64_t whole_groups = n_whole * kCopySplit;
  Piece pc;
  if (grp < whole_groups) {  // a part of a whole piece
    pc = pieces[grp / kCopySplit];
    const int64_t part = (grp % kCopySplit) * kCopyPart;
    pc.shard_off += part;
    pc.canon_off += part;
    pc.len = (int32_t)kCopyPart;
  } else {
    pc = pieces[n_whole + (grp - whole_groups)];
  }
  const int64_t s0 = pc.shard_off, c0 = pc.canon_off;
  const bool vec = al16(master + s0) && al16(mom1 + s0) && al16(mom2 + s0) &&
                   al16(c_master + c0) && al16(c_m + c0) && al16(c_v + c0) &&
                   (EXPORT || ((uintptr_t)(param + s0) & 7u) == 0);
  int32_t done = 0;
  if (vec) {
    const int32_t quads = pc.len >> 2;
    // the part's outputs as buffer resources (uniform over the workgroup), written
    // with the streamed-output store policy
    const int bytes32 = pc.len * 4;
    const __amdgpu_buffer_rsrc_t o1 = out_rsrc(EXPORT ? c_master + c0 : master + s0, bytes32);
    const __amdgpu_buffer_rsrc_t o2 = out_rsrc(EXPORT ? c_m + c0 : mom1 + s0, bytes32);
    const __amdgpu_buffer_rsrc_t o3 = out_rsrc(EXPORT ? c_v + c0 : mom2 + s0, bytes32);
    for (int32_t q = threadIdx.x; q < quads; q += kCopyLanes) {
      const int64_t s = s0 + 4 * (int64_t)q, c = c0 + 4 * (int64_t)q;
      if (EXPORT) {
        const f32x4 a = ld_stream(reinterpret_cast<const f32x4*>(master + s));
        const f32x4 b = ld_stream(reinterpret_cast<const f32x4*>(mom1 + s));
        const f32x4 d = ld_stream(reinterpret_cast<const f32x4*>(mom2 + s));
        st_out(o1, q * 16, a);
        st_out(o2, q * 16, b);
        st_out(o3, q * 16, d);
      } else {
        const f32x4 p = ld_stream(reinterpret_cast<const f32x4*>(c_master + c));
        const f32x4 a = ld_stream(reinterpret_cast<const f32x4*>(c_m + c));
        const f32x4 d = ld_stream(reinterpret_cast<const f32x4*>(c_v + c));
        st_out(o1, q * 16, p);
        st_out(o2, q * 16, a);
        st_out(o3, q * 16, d);
        uint32_t b[4];
#pragma unroll
        for (int k = 0; k < 4; k++) b[k] = F16 ? f2h(p[k]) : to_bf16(p[k]);
        u32x2 pk;
        pk.x = b[0] | (b[1] << 16);
        pk.y = b[2] | (b[3] << 16);
        st_out(out_rsrc(param + s0, pc.len * 2), q * 8, pk);
      }
    }
    done = quads << 2;
    for (int32_t i = done + threadIdx.x; i < pc.len; i += kCopyLanes)
      copy_one<EXPORT, F16>(s0 + i, c0 + i, master, mom1, mom2, param, c_master, c_m, c_v);
    return;
  }
  // 4-byte path: lane t takes elements t, t + 64, t + 128, t + 192 of the part
  // (each access instruction covers 256 contiguous bytes), and issues every
  // load before its first store, so a wave keeps as many bytes in flight as
  // on the 16-byte path.  The fp32 outputs use ordinary stores: an unaligned
  // part shares its first and last cache lines with its neighbours, and
  // measured on MI355X (stress layout, mostly unaligned canonical offsets)
  // export ran 4.72 TB/s this way against 3.93 with non-temporal stores.
  const float* src1 = EXPORT ? master + s0 : c_master + c0;
  const float* src2 = EXPORT ? mom1 + s0 : c_m + c0;
  const float* src3 = EXPORT ? mom2 + s0 : c_v + c0;
  float* dst1 = EXPORT ? c_master + c0 : master + s0;
  float* dst2 = EXPORT ? c_m + c0 : mom1 + s0;
  float* dst3 = EXPORT ? c_v + c0 : mom2 + s0;
  float x1[4], x2[4], x3[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int32_t i = (int32_t)threadIdx.x + k * kCopyLanes;
    if (i < pc.len) {
      x1[k] = ld_stream(src1 + i);
      x2[k] = ld_stream(src2 + i);
      x3[k] = ld_stream(src3 + i);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int32_t i = (int32_t)threadIdx.x + k * kCopyLanes;
    if (i < pc.len) {
      dst1[i] = x1[k];
      dst2[i] = x2[k];
      dst3[i] = x3[k];
      if (!EXPORT)
        __builtin_nontemporal_store((uint16_t)(F16 ? f2h(x1[k]) : to_bf16(x1[k])), param + s0 + i);
    }
  }
}

// ------------------------------------------------- loss-scaled fp16 path
//
// fp16 contributions carry the loss scale; each element's average is unscaled
// by inv_scale = fp32(1/scale) right after the M-way divide.  Found-inf is a
// non-finite sum of squares of the unscaled average (any NaN/Inf element makes
// it so), decided by the finalize step together with the clip coefficient, the
// step constants at t = applied + 1, and the scaler update -- all on the
// device, so a skipped step costs no host round trip.  Conversions use the
// hardware's IEEE fp16 <-> fp32 instructions (exact widening; round to nearest
// even narrowing with overflow to Inf).

template <int M, bool STAGE>
__global__ __launch_bounds__(kThreads) void sumsq_f16_kernel(GradPtrs g, int64_t n,
                                                             double* __restrict__ partials,
                                                             const AmpState* __restrict__ st,
                                                             float* __restrict__ stage,
                                                             int64_t group0) {
  const float inv = (float)(1.0 / (double)st->scale);
  const int64_t blk = group0 + blockIdx.x;
  const int64_t base = blk * kNormTile + (int64_t)threadIdx.x * 4;
  bool in[2];
  u32x2 w[2][M];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int64_t e = base + h * (kNormTile / 2);
    in[h] = e < n;
    if (in[h]) {
#pragma unroll
      for (int j = 0; j < M; j++) w[h][j] = ld_stream(reinterpret_cast<const u32x2*>(g.p[j] + e));
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    if (!in[h]) continue;
    float s[4];
    s[0] = h2f(w[h][0].x); s[1] = h2f(w[h][0].x >> 16);
    s[2] = h2f(w[h][0].y); s[3] = h2f(w[h][0].y >> 16);
#pragma unroll
    for (int j = 1; j < M; j++) {
      s[0] = s[0] + h2f(w[h][j].x); s[1] = s[1] + h2f(w[h][j].x >> 16);
      s[2] = s[2] + h2f(w[h][j].y); s[3] = s[3] + h2f(w[h][j].y >> 16);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      s[q] = (s[q] / (float)M) * inv;
      const double x = (double)s[q];
      acc = acc + x * x;
    }
    if (STAGE) {
      f32x4 a;
      a[0] = s[0]; a[1] = s[1]; a[2] = s[2]; a[3] = s[3];
      st_out(out_rsrc(stage + blk * kNormTile + h * (kNormTile / 2),
                      (int)(kNormTile / 2) * 4),
             threadIdx.x * 16, a);
    }
  }
  const double t = block_sum(acc);
  if (threadIdx.x == 0) partials[blk] = t;
}

// external (nullable): the global sum of squares over every rank's shard, which
// then replaces this shard's partials (the multi-rank split of the step).
__global__ __launch_bounds__(kThreads) void amp_finalize_kernel(
    const double* __restrict__ partials, int32_t n, const double* __restrict__ external,
    AmpState* __restrict__ st, AmpParams p, ClipScalars* __restrict__ out,
    StepConsts* __restrict__ kout) {
  const double part = external ? 0.0 : sum_partials(partials, n);
  if (threadIdx.x != 0) return;
  const double total = external ? *external : part;
  AmpState s = *st;
  const bool found_inf = !__builtin_isfinite(total);
  const double norm = __builtin_sqrt(total);
  float coef = 1.0f;
  if (p.clip) {
    double c = (double)p.max_norm / (norm + 1e-6);
    if (c > 1.0) c = 1.0;
    coef = (float)c;
  }
  ClipScalars r;
  r.sumsq = total;
  r.norm = norm;
  r.coef = coef;
  r.skip = found_inf ? 1u : 0u;
  r.inv_scale = (float)(1.0 / (double)s.scale);
  r.pad = 0;
  *kout = step_consts(p.lr, p.beta1, p.beta2, p.eps, p.weight_decay, s.applied_steps + 1);
  if (found_inf) {
    s.scale = s.scale * p.backoff;
    s.growth_tracker = 0;
  } else {
    s.applied_steps += 1;
    const int32_t good = s.growth_tracker + 1;
    if (good == p.interval) {
      // a grown scale that is not finite is dropped (torch's GradScaler): an
      // Inf scale would unscale every later gradient to zero
      const float grown = s.scale * p.growth;
      if (__builtin_isfinite(grown)) s.scale = grown;
      s.growth_tracker = 0;
    } else {
      s.growth_tracker = good;
    }
  }
  *out = r;
  *st = s;
}

template <int M>
__global__ __launch_bounds__(kStepLanes) void step_f16_kernel(
    GradPtrs g, float* __restrict__ master, float* __restrict__ mom1, float* __restrict__ mom2,
    uint16_t* __restrict__ param, int64_t n, RunTable rt, const ClipScalars* __restrict__ clip,
    const StepConsts* __restrict__ kp, int64_t group0) {
  const int64_t tile = group0 + blockIdx.x;
  const int64_t tile0 = tile * kTile;
  const int64_t e = tile0 + (int64_t)threadIdx.x * kStepVec;
  if (e >= n) return;
  u32x2 w[M];
#pragma unroll
  for (int j = 0; j < M; j++) w[j] = ld_stream(reinterpret_cast<const u32x2*>(g.p[j] + e));
  f32x4 p4 = ld_stream(reinterpret_cast<const f32x4*>(master + e));
  f32x4 m4 = ld_stream(reinterpret_cast<const f32x4*>(mom1 + e));
  f32x4 v4 = ld_stream(reinterpret_cast<const f32x4*>(mom2 + e));
  const uint32_t dflag = decay_flag(rt, tile, tile0, e);
  if (clip->skip) return;  // found-inf: uniform over the grid
  const StepConsts k = *kp;
  const float inv = clip->inv_scale, coef = clip->coef;
  const float d = dflag ? k.decay_mul : 1.0f;
  float s[kStepVec];
  s[0] = h2f(w[0].x); s[1] = h2f(w[0].x >> 16);
  s[2] = h2f(w[0].y); s[3] = h2f(w[0].y >> 16);
#pragma unroll
  for (int j = 1; j < M; j++) {
    s[0] = s[0] + h2f(w[j].x); s[1] = s[1] + h2f(w[j].x >> 16);
    s[2] = s[2] + h2f(w[j].y); s[3] = s[3] + h2f(w[j].y >> 16);
  }
  uint32_t b[kStepVec];
#pragma unroll
  for (int q = 0; q < kStepVec; q++) {
    float gq = (s[q] / (float)M) * inv;
    gq = gq * coef;
    float p = p4[q], m = m4[q], v = v4[q];
    adamw(gq, p, m, v, k, d);
    p4[q] = p;
    m4[q] = m;
    v4[q] = v;
    b[q] = f2h(p);
  }
  u32x2 ph;
  ph.x = b[0] | (b[1] << 16);
  ph.y = b[2] | (b[3] << 16);
  store_step(master, mom1, mom2, param, tile0, p4, m4, v4, ph);
}

__global__ void amp_state_init_kernel(AmpState* st, float scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    AmpState s;
    s.scale = scale;
    s.growth_tracker = 0;
    s.applied_steps = 0;
    *st = s;
  }
}

// The step on a staged average: the norm pass of the same call stored each
// element's averaged (and, for fp16, unscaled) gradient, so this pass reads 4
// bytes of gradient per element instead of the M contributions.  The values
// are the very bits the fused kernels recompute, so results are identical.
// AMP: constants from the device (loss-scaled path), fp16 param; otherwise the
// host's constants and a bf16 param.
template <bool AMP>
__global__ __launch_bounds__(kStepLanes) void step_staged_kernel(
    const float* __restrict__ stage, float* __restrict__ master, float* __restrict__ mom1,
    float* __restrict__ mom2, uint16_t* __restrict__ param, int64_t n, RunTable rt,
    const ClipScalars* __restrict__ clip, StepConsts kh, const StepConsts* __restrict__ kd,
    int64_t group0) {
  const int64_t tile = group0 + blockIdx.x;
  const int64_t tile0 = tile * kTile;
  const int64_t e = tile0 + (int64_t)threadIdx.x * kStepVec;
  if (e >= n) return;
  f32x4 g4 = ld_stream(reinterpret_cast<const f32x4*>(stage + e));
  f32x4 p4 = ld_stream(reinterpret_cast<const f32x4*>(master + e));
  f32x4 m4 = ld_stream(reinterpret_cast<const f32x4*>(mom1 + e));
  f32x4 v4 = ld_stream(reinterpret_cast<const f32x4*>(mom2 + e));
  const uint32_t dflag = decay_flag(rt, tile, tile0, e);
  if (clip->skip) return;  // uniform over the grid
  const StepConsts k = AMP ? *kd : kh;
  const float coef = clip->coef;  // 1 when the call does not clip
  const float d = dflag ? k.decay_mul : 1.0f;
  uint32_t b[kStepVec];
#pragma unroll
  for (int q = 0; q < kStepVec; q++) {
    const float gq = g4[q] * coef;
    float p = p4[q], m = m4[q], v = v4[q];
    adamw(gq, p, m, v, k, d);
    p4[q] = p;
    m4[q] = m;
    v4[q] = v;
    b[q] = AMP ? f2h(p) : to_bf16(p);
  }
  u32x2 pk;
  pk.x = b[0] | (b[1] << 16);
  pk.y = b[2] | (b[3] << 16);
  store_step(master, mom1, mom2, param, tile0, p4, m4, v4, pk);
}

// A dispatch carries at most 2^32 - 1 work-items (its grid size is a 32-bit
// count of work-items), which a step grid passes beyond 2^34 elements.  Larger
// grids go out as consecutive slices of whole work-groups on the same stream;
// launch(group0, groups) issues one slice and its kernel adds group0 to
// blockIdx.x.  max_groups > 0 lowers the slice size.
template <typename F>
hipError_t for_slices(int64_t groups, int block, int64_t max_groups, F&& launch) {
  const int64_t lim = (int64_t)0xffffffff / block;
  const int64_t per = (max_groups > 0 && max_groups < lim) ? max_groups : lim;
  for (int64_t g0 = 0; g0 < groups; g0 += per) {
    launch(g0, (unsigned)(groups - g0 < per ? groups - g0 : per));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int M>
hipError_t launch_sumsq_f16_m(const GradPtrs& g, int64_t shard_len, double* partials,
                              const AmpState* st, float* stage, size_t stage_lds,
                              int64_t max_groups, hipStream_t stream) {
  const int64_t p1 = (shard_len + kNormTile - 1) / kNormTile;
  const hipError_t e = for_slices(p1, kThreads, max_groups, [&](int64_t g0, unsigned n) {
    if (stage)
      hipLaunchKernelGGL((sumsq_f16_kernel<M, true>), dim3(n), dim3(kThreads), stage_lds,
                         stream, g, shard_len, partials, st, stage, g0);
    else
      hipLaunchKernelGGL((sumsq_f16_kernel<M, false>), dim3(n), dim3(kThreads), 0, stream, g,
                         shard_len, partials, st, stage, g0);
  });
  if (e != hipSuccess) return e;
  const int64_t p2 = (p1 + kLevel2 - 1) / kLevel2;
  hipLaunchKernelGGL(sum_blocks_kernel, dim3((unsigned)p2), dim3(kThreads), 0, stream,
                     partials, p1, partials + p1);
  return hipGetLastError();
}

template <int M>
hipError_t launch_step_f16_m(const GradPtrs& g, float* master, float* m, float* v,
                             uint16_t* param, int64_t n, const RunTable& rt,
                             const ClipScalars* clip, const StepConsts* k, size_t lds,
                             int64_t max_groups, hipStream_t stream) {
  const int64_t tiles = (n + kTile - 1) / kTile;
  return for_slices(tiles, kStepLanes, max_groups, [&](int64_t g0, unsigned nt) {
    hipLaunchKernelGGL((step_f16_kernel<M>), dim3(nt), dim3(kStepLanes), lds, stream, g, master,
                       m, v, param, n, rt, clip, k, g0);
  });
}

template <int M>
hipError_t launch_step_m(bool use_clip, const GradPtrs& g, float* master, float* m, float* v,
                         uint16_t* param, int64_t n, const RunTable& rt,
                         const ClipScalars* clip, const StepConsts& k, size_t lds,
                         int64_t max_groups, hipStream_t stream) {
  const int64_t tiles = (n + kTile - 1) / kTile;
  return for_slices(tiles, kStepLanes, max_groups, [&](int64_t g0, unsigned nt) {
    if (use_clip)
      hipLaunchKernelGGL((step_kernel<M, true>), dim3(nt), dim3(kStepLanes), lds, stream, g,
                         master, m, v, param, n, rt, clip, k, g0);
    else
      hipLaunchKernelGGL((step_kernel<M, false>), dim3(nt), dim3(kStepLanes), lds, stream, g,
                         master, m, v, param, n, rt, clip, k, g0);
  });
}

template <int M>
hipError_t launch_sumsq_m(const GradPtrs& g, int64_t shard_len, double* partials, float* stage,
                          size_t stage_lds, int64_t max_groups, hipStream_t stream) {
  const int64_t p1 = (shard_len + kNormTile - 1) / kNormTile;
  const hipError_t e = for_slices(p1, kThreads, max_groups, [&](int64_t g0, unsigned n) {
    if (stage)
      hipLaunchKernelGGL((sumsq_kernel<M, true>), dim3(n), dim3(kThreads), stage_lds, stream,
                         g, shard_len, partials, stage, g0);
    else
      hipLaunchKernelGGL((sumsq_kernel<M, false>), dim3(n), dim3(kThreads), 0, stream, g,
                         shard_len, partials, stage, g0);
  });
  if (e != hipSuccess) return e;
  const int64_t p2 = (p1 + kLevel2 - 1) / kLevel2;
  hipLaunchKernelGGL(sum_blocks_kernel, dim3((unsigned)p2), dim3(kThreads), 0, stream,
                     partials, p1, partials + p1);
  return hipGetLastError();
}

// Small host tables handed to the device through kernel arguments: each
// launch carries up to kArgWords 32-bit words by value and one workgroup
// stores them.  No host memory is read once the launch call has returned,
// nothing is allocated, and the launches can be captured in a graph.
constexpr int kArgWords = 512;  // 2 KiB of payload, well inside the kernel-argument limit
struct ArgWords {
  uint32_t w[kArgWords];
};

__global__ __launch_bounds__(kThreads) void store_words_kernel(ArgWords a,
                                                               uint32_t* __restrict__ dst,
                                                               int32_t n) {
  for (int32_t i = threadIdx.x; i < n; i += kThreads) dst[i] = a.w[i];
}

// The tile-flag table from a run table on the device (the same 2 bits per
// step tile the planner computes on the host): thread w builds word w, tiles
// 16w .. 16w + 15.  runs[n_runs] is the sentinel (start = shard_len), and
// runs[0].start == 0, so every tile's first element lies in some run.
__global__ __launch_bounds__(kThreads) void tile_flags_kernel(const Run* __restrict__ runs,
                                                              int32_t n_runs, int64_t shard_len,
                                                              uint32_t* __restrict__ flags,
                                                              int64_t words) {
  const int64_t wi = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (wi >= words) return;
  const int64_t tiles = (shard_len + kTile - 1) / kTile;
  uint32_t out = 0;
  for (int k = 0; k < 16; k++) {
    const int64_t t = wi * 16 + k;
    if (t >= tiles) break;
    const int64_t lo = t * kTile;
    const int64_t hi = lo + kTile < shard_len ? lo + kTile : shard_len;
    const int32_t r = find_run(runs, n_runs, lo);
    const uint32_t f = runs[r + 1].start < hi ? 2u : ((uint32_t)runs[r].flags & 1u);
    out |= f << (k * 2);
  }
  flags[wi] = out;
}

}  // namespace

hipError_t launch_store_words(const uint32_t* host_words, int64_t n_words, uint32_t* dst,
                              hipStream_t stream) {
  for (int64_t off = 0; off < n_words; off += kArgWords) {
    ArgWords a;
    const int32_t m = (int32_t)(n_words - off < kArgWords ? n_words - off : kArgWords);
    for (int32_t i = 0; i < kArgWords; i++) a.w[i] = i < m ? host_words[off + i] : 0u;
    hipLaunchKernelGGL(store_words_kernel, dim3(1), dim3(kThreads), 0, stream, a, dst + off, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_tile_flags(const Run* runs, int32_t n_runs, int64_t shard_len, uint32_t* flags,
                             hipStream_t stream) {
  const int64_t words = tile_flag_words(shard_len, n_runs);
  if (words <= 0) return hipSuccess;
  const int64_t blocks = (words + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_flags_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, runs,
                     n_runs, shard_len, flags, words);
  return hipGetLastError();
}

// Level-1 plus level-2 partials of the norm pass; the level-2 ones (at most a few
// thousand) start at offset level1_partials(shard_len) and feed the finalize step.
int64_t level1_partials(int64_t shard_len) {
  const int64_t p1 = (shard_len + kNormTile - 1) / kNormTile;
  return p1 > 0 ? p1 : 1;
}

int64_t sumsq_partials(int64_t shard_len) {
  const int64_t p1 = level1_partials(shard_len);
  return p1 + (p1 + kLevel2 - 1) / kLevel2;
}

int32_t final_partials(int64_t shard_len) {
  return (int32_t)((level1_partials(shard_len) + kLevel2 - 1) / kLevel2);
}

#define ZS_DISPATCH_M(M_, CALL) \
  switch (M_) {                 \
    case 1: return CALL(1);     \
    case 2: return CALL(2);     \
    case 3: return CALL(3);     \
    case 4: return CALL(4);     \
    case 5: return CALL(5);     \
    case 6: return CALL(6);     \
    case 7: return CALL(7);     \
    case 8: return CALL(8);     \
    case 9: return CALL(9);     \
    case 10: return CALL(10);   \
    case 11: return CALL(11);   \
    case 12: return CALL(12);   \
    case 13: return CALL(13);   \
    case 14: return CALL(14);   \
    case 15: return CALL(15);   \
    case 16: return CALL(16);   \
    default: return hipErrorInvalidValue; \
  }

// A step launch needs its run data: a run table, and the tile flags when there
// is more than one run.
static bool step_args_ok(const RunTable& rt) {
  return rt.n_runs >= 1 && rt.runs && (rt.n_runs == 1 || rt.tile_flags);
}

hipError_t launch_step(int M, bool use_clip, const GradPtrs& g, float* master, float* m,
                       float* v, uint16_t* param, int64_t shard_len, const RunTable& rt,
                       const ClipScalars* clip, const StepConsts& k, size_t lds,
                       int64_t max_groups, hipStream_t stream) {
  if (shard_len <= 0) return hipSuccess;
  if (!step_args_ok(rt)) return hipErrorInvalidValue;
#define ZS_CALL_STEP(X) \
  launch_step_m<X>(use_clip, g, master, m, v, param, shard_len, rt, clip, k, lds, max_groups, \
                   stream)
  ZS_DISPATCH_M(M, ZS_CALL_STEP)
#undef ZS_CALL_STEP
}

hipError_t launch_sumsq(int M, const GradPtrs& g, int64_t shard_len, double* partials,
                        float* stage, size_t stage_lds, int64_t max_groups, hipStream_t stream) {
  if (shard_len <= 0 || level1_partials(shard_len) > 0x7fffffff) return hipErrorInvalidValue;
#define ZS_CALL_SUMSQ(X) \
  launch_sumsq_m<X>(g, shard_len, partials, stage, stage_lds, max_groups, stream)
  ZS_DISPATCH_M(M, ZS_CALL_SUMSQ)
#undef ZS_CALL_SUMSQ
}

hipError_t launch_state_copy(bool do_export, bool param_f16, const Piece* pieces,
                             int64_t n_pieces, int64_t n_whole, float* master, float* m, float* v,
                             uint16_t* param, float* c_master, float* c_m, float* c_v,
                             size_t lds, int64_t max_groups, hipStream_t stream) {
  if (n_pieces <= 0) return hipSuccess;
  if (n_whole < 0 || n_whole > n_pieces) return hipErrorInvalidValue;
  const dim3 block(kCopyLanes);
  const int64_t groups = n_whole * kCopySplit + (n_pieces - n_whole);
  return for_slices(groups, kCopyLanes, max_groups, [&](int64_t g0, unsigned n) {
    if (do_export)
      hipLaunchKernelGGL((state_copy_kernel<true, false>), dim3(n), block, lds, stream, pieces,
                         n_whole, master, m, v, param, c_master, c_m, c_v, g0);
    else if (param_f16)
      hipLaunchKernelGGL((state_copy_kernel<false, true>), dim3(n), block, lds, stream, pieces,
                         n_whole, master, m, v, param, c_master, c_m, c_v, g0);
    else
      hipLaunchKernelGGL((state_copy_kernel<false, false>), dim3(n), block, lds, stream, pieces,
                         n_whole, master, m, v, param, c_master, c_m, c_v, g0);
  });
}

hipError_t launch_sumsq_f16(int M, const GradPtrs& g, int64_t shard_len, double* partials,
                            const AmpState* st, float* stage, size_t stage_lds,
                            int64_t max_groups, hipStream_t stream) {
  if (shard_len <= 0 || level1_partials(shard_len) > 0x7fffffff) return hipErrorInvalidValue;
#define ZS_CALL_SUMSQ16(X) \
  launch_sumsq_f16_m<X>(g, shard_len, partials, st, stage, stage_lds, max_groups, stream)
  ZS_DISPATCH_M(M, ZS_CALL_SUMSQ16)
#undef ZS_CALL_SUMSQ16
}

hipError_t launch_amp_finalize(const double* partials, int32_t n_partials,
                               const double* external, AmpState* st, const AmpParams& p,
                               ClipScalars* out, StepConsts* kout, hipStream_t stream) {
  hipLaunchKernelGGL(amp_finalize_kernel, dim3(1), dim3(kThreads), 0, stream, partials,
                     n_partials, external, st, p, out, kout);
  return hipGetLastError();
}

hipError_t launch_step_f16(int M, const GradPtrs& g, float* master, float* m, float* v,
                           uint16_t* param, int64_t shard_len, const RunTable& rt,
                           const ClipScalars* clip, const StepConsts* k, size_t lds,
                           int64_t max_groups, hipStream_t stream) {
  if (shard_len <= 0) return hipSuccess;
  if (!step_args_ok(rt)) return hipErrorInvalidValue;
#define ZS_CALL_STEP16(X) \
  launch_step_f16_m<X>(g, master, m, v, param, shard_len, rt, clip, k, lds, max_groups, stream)
  ZS_DISPATCH_M(M, ZS_CALL_STEP16)
#undef ZS_CALL_STEP16
}

hipError_t launch_step_staged(bool amp, const float* stage, float* master, float* m, float* v,
                              uint16_t* param, int64_t shard_len, const RunTable& rt,
                              const ClipScalars* clip, const StepConsts& kh, const StepConsts* kd,
                              size_t lds, int64_t max_groups, hipStream_t stream) {
  if (shard_len <= 0) return hipSuccess;
  if (!step_args_ok(rt)) return hipErrorInvalidValue;
  const int64_t tiles = (shard_len + kTile - 1) / kTile;
  return for_slices(tiles, kStepLanes, max_groups, [&](int64_t g0, unsigned nt) {
    if (amp)
      hipLaunchKernelGGL((step_staged_kernel<true>), dim3(nt), dim3(kStepLanes), lds, stream,
                         stage, master, m, v, param, shard_len, rt, clip, kh, kd, g0);
    else
      hipLaunchKernelGGL((step_staged_kernel<false>), dim3(nt), dim3(kStepLanes), lds, stream,
                         stage, master, m, v, param, shard_len, rt, clip, kh, kd, g0);
  });
}

hipError_t launch_amp_state_init(AmpState* st, float scale, hipStream_t stream) {
  hipLaunchKernelGGL(amp_state_init_kernel, dim3(1), dim3(64), 0, stream, st, scale);
  return hipGetLastError();
}

hipError_t launch_finalize(const double* partials, int32_t n_partials,
                           const double* external_sumsq, float max_norm, int clip,
                           int skip_nonfinite, ClipScalars* out, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kThreads), 0, stream, partials, n_partials,
                     external_sumsq, max_norm, clip, skip_nonfinite, out);
  return hipGetLastError();
}

hipError_t launch_sumsq_total(const double* partials, int32_t n_partials, double* out,
                              hipStream_t stream) {
  hipLaunchKernelGGL(sumsq_total_kernel, dim3(1), dim3(kThreads), 0, stream, partials,
                     n_partials, out);
  return hipGetLastError();
}

namespace {

hipError_t static_lds_of(const void* kernel, size_t* worst) {
  hipFuncAttributes a{};
  const hipError_t e = hipFuncGetAttributes(&a, kernel);
  if (e == hipSuccess && a.sharedSizeBytes > *worst) *worst = a.sharedSizeBytes;
  return e;
}

template <int M>
hipError_t static_lds_m(size_t* worst) {
  const void* k[] = {reinterpret_cast<const void*>(&step_kernel<M, false>),
                     reinterpret_cast<const void*>(&step_kernel<M, true>),
                     reinterpret_cast<const void*>(&step_f16_kernel<M>),
                     reinterpret_cast<const void*>(&sumsq_kernel<M, true>),
                     reinterpret_cast<const void*>(&sumsq_f16_kernel<M, true>),
                     reinterpret_cast<const void*>(&step_staged_kernel<false>),
                     reinterpret_cast<const void*>(&step_staged_kernel<true>),
                     reinterpret_cast<const void*>(&state_copy_kernel<true, false>),
                     reinterpret_cast<const void*>(&state_copy_kernel<false, false>),
                     reinterpret_cast<const void*>(&state_copy_kernel<false, true>)};
  for (const void* f : k) {
    const hipError_t e = static_lds_of(f, worst);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t reserved_kernels_static_lds(int M, size_t* worst) {
  *worst = 0;
#define ZS_CALL_STATIC(X) static_lds_m<X>(worst)
  ZS_DISPATCH_M(M, ZS_CALL_STATIC)
#undef ZS_CALL_STATIC
}

}  // namespace zs
