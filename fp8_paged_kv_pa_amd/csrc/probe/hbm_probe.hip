// Streaming-read bandwidth probe for MI355X: every lane reads 16-byte
// vectors of a large buffer with a grid-stride loop and folds them into one
// word per thread, so the only traffic is the read (and a tiny write).
// Used by the bench as the measured companion of the 8 TB/s HBM peak (a
// bench-only library, not part of the C ABI).
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

// Block-read probe: the access pattern of a one-row decode without its
// arithmetic.  Workgroup w reads the (page, head) blocks listed in
// table[w*per_wg .. (w+1)*per_wg): 16 KiB of K and 16 KiB of V per entry,
// plus, with scales, that block's 512-byte K and V scale pieces (read by
// half a wave), all with non-temporal 16-byte loads, two entries in flight.
// It measures what streaming exactly those blocks costs, the ceiling the
// decode's memory traffic meets.
__global__ __launch_bounds__(256) void hbm_block_kernel(const u32x4* __restrict__ kp, const u32x4* __restrict__ vp,
                                                        const u32x4* __restrict__ ksp, const u32x4* __restrict__ vsp,
                                                        const int32_t* __restrict__ table, int per_wg,
                                                        uint32_t* __restrict__ sink) {
  const int32_t* t = table + int64_t(blockIdx.x) * per_wg;
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  for (int n = 0; n < per_wg; n += 2) {
    const int m = (n + 1 < per_wg) ? n + 1 : n;
    const int64_t b0 = int64_t(t[n]) * 1024, b1 = int64_t(t[m]) * 1024;  // blocks in 16-byte units
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = __builtin_nontemporal_load(&kp[b0 + k * 256 + tid]);
      v[4 + k] = __builtin_nontemporal_load(&vp[b0 + k * 256 + tid]);
      v[8 + k] = __builtin_nontemporal_load(&kp[b1 + k * 256 + tid]);
      v[12 + k] = __builtin_nontemporal_load(&vp[b1 + k * 256 + tid]);
    }
    if (ksp && tid < 32) {
      const u32x4 a = __builtin_nontemporal_load(&ksp[int64_t(t[n]) * 32 + tid]);
      const u32x4 b = __builtin_nontemporal_load(&vsp[int64_t(t[n]) * 32 + tid]);
      const u32x4 c = __builtin_nontemporal_load(&ksp[int64_t(t[m]) * 32 + tid]);
      const u32x4 d = __builtin_nontemporal_load(&vsp[int64_t(t[m]) * 32 + tid]);
      acc ^= a.x ^ b.y ^ c.z ^ d.w;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  sink[int64_t(blockIdx.x) * blockDim.x + tid] = acc;
}

// k_cache, v_cache: FP8 blocks of 16 KiB ([num_blocks*Hkv, 16384] bytes);
// k_scale, v_scale: their fp32 [num_blocks*Hkv, 128] scales, or both NULL;
// table: int32 [wgs * per_wg] block ids, each in [0, num_blocks*Hkv) (the
// caller checks); sink: wgs*256 uint32.
extern "C" int hbm_block_probe(const void* k_cache, const void* v_cache, const void* k_scale,
                               const void* v_scale, const int32_t* table, int per_wg, int wgs, void* sink,
                               void* stream) {
  if (!k_cache || !v_cache || !table || !sink || per_wg < 1 || wgs < 1) return -1;
  if ((k_scale == nullptr) != (v_scale == nullptr)) return -1;
  hipLaunchKernelGGL(hbm_block_kernel, dim3(wgs), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(k_cache), static_cast<const u32x4*>(v_cache),
                     static_cast<const u32x4*>(k_scale), static_cast<const u32x4*>(v_scale), table, per_wg,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
