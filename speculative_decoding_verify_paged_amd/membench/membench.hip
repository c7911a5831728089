// membench.hip — libpa_membench.so: the two reference kernels the
// measurements need next to the attention kernels.
//   pa_membench_read: streams a buffer once with 16-byte nontemporal loads (the HBM read
//     ceiling the attention kernel's bandwidth is compared with).
//   pa_membench_copy: copies a buffer of known size (calibrates the
//     FETCH_SIZE / WRITE_SIZE counters into bytes).
// Measurement tools only; the attention path does not use them.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void membench_read(const u32x4* __restrict__ p, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9e3779b9u) sink[blockIdx.x] = r;   // keeps the loads alive; practically never stores
}

__global__ __launch_bounds__(256) void membench_copy(u32x4* __restrict__ dst,
                                                     const u32x4* __restrict__ src, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

extern "C" {

// bytes must be a multiple of 16; grid workgroups of 256 threads.
int pa_membench_read(const void* buf, size_t bytes, void* sink, int grid, void* stream) {
  if (!buf || !sink || bytes % 16 || grid < 1) return 1;
  const u32x4* b = (const u32x4*)buf;
  size_t n = bytes / 16;
  uint32_t* k = (uint32_t*)sink;
  void* args[] = {&b, &n, &k};
  return hipLaunchKernel(reinterpret_cast<const void*>(membench_read), dim3(grid), dim3(256), args,
                         0, (hipStream_t)stream) == hipSuccess ? 0 : 4;
}

int pa_membench_copy(void* dst, const void* src, size_t bytes, int grid, void* stream) {
  if (!dst || !src || bytes % 16 || grid < 1) return 1;
  u32x4* d = (u32x4*)dst;
  const u32x4* s = (const u32x4*)src;
  size_t n = bytes / 16;
  void* args[] = {&d, &s, &n};
  return hipLaunchKernel(reinterpret_cast<const void*>(membench_copy), dim3(grid), dim3(256), args,
                         0, (hipStream_t)stream) == hipSuccess ? 0 : 4;
}

}  // extern "C"
