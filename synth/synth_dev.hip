// synth_dev.hip -- seeded synthetic inputs made directly in device memory.
//
// Test and benchmark infrastructure, not part of the optimizer path.  The
// definition (splitmix64 counter hash, Irwin-Hall approximate normal, bf16 by
// truncation, gradient kinds from a second stream) is the one written out in
// synth_host.c; both sides give identical bits for every index.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t hash_at(uint64_t key, uint64_t i) {
  return mix(key + (i + 1) * kGolden);
}

__device__ __forceinline__ float normal_f32(uint64_t h, float scale) {
  int32_t s = (int32_t)(h & 0xffff) + (int32_t)((h >> 16) & 0xffff) +
              (int32_t)((h >> 32) & 0xffff) + (int32_t)(h >> 48);
  return (float)(s - 131070) * scale;
}

__device__ __forceinline__ uint16_t upper16(float x) {
  return (uint16_t)(__float_as_uint(x) >> 16);
}

struct Kinds {
  uint32_t zero_ppm, subnormal_ppm, outlier_ppm;
};

__device__ __forceinline__ uint16_t grad_bf16(uint64_t key, uint64_t ksel,
                                              uint64_t i, float scale,
                                              float out_scale, Kinds k) {
  if (k.zero_ppm | k.subnormal_ppm | k.outlier_ppm) {
    uint64_t sel = hash_at(ksel, i);
    uint32_t r = (uint32_t)((sel >> 32) % 1000000u);
    if (r < k.zero_ppm) return 0;
    r -= k.zero_ppm;
    if (r < k.subnormal_ppm)
      return (uint16_t)((((sel >> 31) & 1u) << 15) |
                        (1u + (uint32_t)((sel >> 8) % 127u)));
    r -= k.subnormal_ppm;
    if (r < k.outlier_ppm) return upper16(normal_f32(hash_at(key, i), out_scale));
  }
  return upper16(normal_f32(hash_at(key, i), scale));
}

// fp32 -> fp16 by truncation (generator only; see synth_host.c).
__device__ __forceinline__ uint16_t trunc_f16(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x47800000u) return (uint16_t)(sign | 0x7c00u);
  if (a < 0x38800000u) return sign;
  return (uint16_t)(sign | ((a - 0x38000000u) >> 13));
}

__global__ void k_grad_f16(uint16_t* out, int64_t n, uint64_t key, int64_t base, float scale,
                           float loss_scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = trunc_f16(normal_f32(hash_at(key, (uint64_t)(base + i)), scale) * loss_scale);
}

__global__ void k_normal_f32(float* out, int64_t n, uint64_t key, int64_t base,
                             float scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    out[i] = normal_f32(hash_at(key, (uint64_t)(base + i)), scale);
}

__global__ void k_grad_bf16(uint16_t* out, int64_t n, uint64_t key,
                            uint64_t ksel, int64_t base, float scale,
                            float out_scale, Kinds kinds) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    out[i] = grad_bf16(key, ksel, (uint64_t)(base + i), scale, out_scale, kinds);
}

// ranges: n_ranges pairs {offset, length} in elements; one workgroup per range.
template <typename T>
__global__ void k_zero_ranges(T* buf, const int64_t* ranges, int64_t n_ranges) {
  int64_t r = blockIdx.x;
  if (r >= n_ranges) return;
  int64_t off = ranges[2 * r], len = ranges[2 * r + 1];
  for (int64_t i = threadIdx.x; i < len; i += blockDim.x) buf[off + i] = T(0);
}

// out[i] = src[idx[i]]: gathers sampled elements for host-side checks.
template <typename T>
__global__ void k_gather(T* out, const T* src, const int64_t* idx, int64_t n) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    out[i] = src[idx[i]];
}

// dst[idx[i]] = src[i]: scatters host-chosen values into sampled elements.
template <typename T>
__global__ void k_scatter(T* dst, const T* src, const int64_t* idx, int64_t n) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    dst[idx[i]] = src[i];
}

// A plain copy of known size, used to calibrate the byte counters.
__global__ void k_copy_u32x4(uint4* dst, const uint4* src, int64_t n) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    dst[i] = src[i];
}

constexpr int kThreads = 256;

unsigned grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

int synth_dev_normal_f32(float* out, int64_t n, uint64_t key, int64_t base,
                         float scale, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(kThreads), 0,
                     (hipStream_t)stream, out, n, key, base, scale);
  return (int)hipGetLastError();
}

int synth_dev_grad_bf16(uint16_t* out, int64_t n, uint64_t key, uint64_t ksel,
                        int64_t base, float scale, float out_scale,
                        uint32_t zero_ppm, uint32_t subnormal_ppm,
                        uint32_t outlier_ppm, void* stream) {
  if (n <= 0) return 0;
  Kinds k{zero_ppm, subnormal_ppm, outlier_ppm};
  hipLaunchKernelGGL(k_grad_bf16, dim3(grid_for(n)), dim3(kThreads), 0,
                     (hipStream_t)stream, out, n, key, ksel, base, scale,
                     out_scale, k);
  return (int)hipGetLastError();
}

int synth_dev_grad_f16(uint16_t* out, int64_t n, uint64_t key, int64_t base, float scale,
                       float loss_scale, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_grad_f16, dim3(grid_for(n)), dim3(kThreads), 0, (hipStream_t)stream, out,
                     n, key, base, scale, loss_scale);
  return (int)hipGetLastError();
}

// elem_bytes: 2 or 4.  ranges is a device array of 2*n_ranges int64.
int synth_dev_zero_ranges(void* buf, int32_t elem_bytes, const int64_t* ranges,
                          int64_t n_ranges, void* stream) {
  if (n_ranges <= 0) return 0;
  if (n_ranges > 0x7fffffff) return -1;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_zero_ranges<uint16_t>, dim3((unsigned)n_ranges),
                       dim3(64), 0, (hipStream_t)stream, (uint16_t*)buf, ranges,
                       n_ranges);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(k_zero_ranges<uint32_t>, dim3((unsigned)n_ranges),
                       dim3(64), 0, (hipStream_t)stream, (uint32_t*)buf, ranges,
                       n_ranges);
  else
    return -1;
  return (int)hipGetLastError();
}

int synth_dev_gather(void* out, const void* src, int32_t elem_bytes,
                     const int64_t* idx, int64_t n, void* stream) {
  if (n <= 0) return 0;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_gather<uint16_t>, dim3(grid_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint16_t*)out, (const uint16_t*)src,
                       idx, n);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(k_gather<uint32_t>, dim3(grid_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint32_t*)out, (const uint32_t*)src,
                       idx, n);
  else
    return -1;
  return (int)hipGetLastError();
}

int synth_dev_scatter(void* dst, const void* src, int32_t elem_bytes,
                      const int64_t* idx, int64_t n, void* stream) {
  if (n <= 0) return 0;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_scatter<uint16_t>, dim3(grid_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint16_t*)dst, (const uint16_t*)src,
                       idx, n);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(k_scatter<uint32_t>, dim3(grid_for(n)), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint32_t*)dst, (const uint32_t*)src,
                       idx, n);
  else
    return -1;
  return (int)hipGetLastError();
}

// Copies n16 16-byte words.  Both pointers must be 16-byte aligned.
int synth_dev_copy16(void* dst, const void* src, int64_t n16, void* stream) {
  if (n16 <= 0) return 0;
  hipLaunchKernelGGL(k_copy_u32x4, dim3(grid_for(n16)), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint4*)dst, (const uint4*)src, n16);
  return (int)hipGetLastError();
}

}  // extern "C"
