// Streaming-read bandwidth probe for MI355X: every lane reads 16-byte
// vectors of a large buffer with a grid-stride loop and folds them into one
// word per thread, so the only traffic is the read (and a tiny write).
// Used by the bench as the measured companion of the 8 TB/s HBM peak.
#include <hip/hip_runtime.h>

#include <cstdint>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                       uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// Read `bytes` (a multiple of 16) from device buffer `src` with `blocks`
// workgroups of 256 threads; `sink` must hold blocks*256 uint32.
extern "C" int hbm_read_probe(const void* src, int64_t bytes, void* sink, int blocks, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes % 16) || blocks < 1) return -1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
