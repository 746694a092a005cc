// The bench's probes for MI355X (a bench-only library, not part of the C
// ABI): the streaming read and the block read below measure what the memory
// system gives the decode's access patterns (the measured companions of the
// 8 TB/s HBM peak); the launch-floor and instruction-rate probes at the end
// measure what any launch costs and what one wave64 instruction of each kind
// the decode issues costs.
//
// Streaming read: every lane reads 16-byte vectors of a large buffer with a
// grid-stride loop and folds them into one word per thread, so the only
// traffic is the read (and a tiny write).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

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
// workgroups of 256 threads; `sink` must hold blocks*256 uint32.  With
// events (both or neither), the dispatch records them at the start and end
// of this kernel, as the decode's main kernel is timed.
extern "C" int hbm_read_probe(const void* src, int64_t bytes, void* sink, int blocks, void* ev_begin,
                              void* ev_end, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes % 16) || blocks < 1 || (ev_begin == nullptr) != (ev_end == nullptr))
    return -1;
  hipExtLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                        reinterpret_cast<hipEvent_t>(ev_begin), reinterpret_cast<hipEvent_t>(ev_end), 0,
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
// caller checks); sink: wgs*256 uint32; events as for hbm_read_probe.
extern "C" int hbm_block_probe(const void* k_cache, const void* v_cache, const void* k_scale,
                               const void* v_scale, const int32_t* table, int per_wg, int wgs, void* sink,
                               void* ev_begin, void* ev_end, void* stream) {
  if (!k_cache || !v_cache || !table || !sink || per_wg < 1 || wgs < 1) return -1;
  if ((k_scale == nullptr) != (v_scale == nullptr) || (ev_begin == nullptr) != (ev_end == nullptr)) return -1;
  hipExtLaunchKernelGGL(hbm_block_kernel, dim3(wgs), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                        reinterpret_cast<hipEvent_t>(ev_begin), reinterpret_cast<hipEvent_t>(ev_end), 0,
                        static_cast<const u32x4*>(k_cache), static_cast<const u32x4*>(v_cache),
                        static_cast<const u32x4*>(k_scale), static_cast<const u32x4*>(v_scale), table, per_wg,
                        static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// ---------------------------------------------------------------------------
// Launch-floor probe: a kernel that does nothing (one branch on a value it
// never sees), so its dispatch-recorded duration is what any launch costs on
// the box, for a grid and block of the caller's choice.
__global__ void empty_kernel(const uint32_t* __restrict__ flag, uint32_t* __restrict__ sink) {
  if (flag[0] == 0x5EEDu && threadIdx.x == 0) sink[blockIdx.x] = 1u;
}

// `flag` and `sink`: device buffers of >= 1 and >= blocks uint32.  With
// events, the dispatch records them (start and end of this kernel), as the
// decode's main kernel is timed.
extern "C" int launch_floor_probe(const void* flag, void* sink, int blocks, int threads, void* ev_begin,
                                  void* ev_end, void* stream) {
  if (!flag || !sink || blocks < 1 || threads < 1 || threads > 1024) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* f = static_cast<const uint32_t*>(flag);
  uint32_t* k = static_cast<uint32_t*>(sink);
  if (ev_begin || ev_end)
    hipExtLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, s, reinterpret_cast<hipEvent_t>(ev_begin),
                          reinterpret_cast<hipEvent_t>(ev_end), 0, f, k);
  else
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, s, f, k);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Workgroup start spread: every workgroup's first wave records the constant
// 100 MHz count (s_memrealtime) on entry; the spread of those counts over a
// launch is how far apart the dispatcher starts its workgroups.  Dynamic
// LDS of the caller's size (and the LDS it forces per CU) is requested
// without being used.
__global__ void start_kernel(long long* __restrict__ ticks) {
  const long long t = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) ticks[blockIdx.x] = t;
}

// `ticks`: device int64 [blocks]; lds_bytes <= 160 KiB.
extern "C" int start_spread_probe(void* ticks, int blocks, int threads, int lds_bytes, void* stream) {
  if (!ticks || blocks < 1 || threads < 64 || threads > 1024 || lds_bytes < 0 || lds_bytes > 160 * 1024)
    return -1;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&start_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          lds_bytes) != hipSuccess)
    return -2;
  hipLaunchKernelGGL(start_kernel, dim3(blocks), dim3(threads), size_t(lds_bytes),
                     reinterpret_cast<hipStream_t>(stream), static_cast<long long*>(ticks));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// ---------------------------------------------------------------------------
// Instruction-rate probe: one or two waves per SIMD (four- or eight-wave
// workgroups, one per CU through a large LDS request) run `iters` rounds
// of independent instructions of one kind; each wave records its
// shader-clock cycles (s_memtime) and the constant 100 MHz count
// (s_memrealtime) over the same interval.  With n waves per SIMD,
// cycles / (iters * per_round * n) is the SIMD's cost per wave64
// instruction of that kind, and cycles / ticks the clock it ran at:
//   kind 0: v_mfma_f32_16x16x32_bf16, 8 per round (8 accumulator chains)
//   kind 1: fp32 fma (v_fmac_f32, 4-byte form), 32 per round (32 chains)
//   kind 2: v_cvt_scalef32_pk_bf16_fp8, 16 per round
//   kind 3: v_exp_f32, 32 per round
//   kind 4 (two waves per SIMD only): the SIMD's first wave runs kind 0's
//          rounds, its second wave four times as many of kind 1's, to show
//          how far the two pipes overlap
typedef __bf16 pb_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pb_bf16x2 __attribute__((ext_vector_type(2)));
typedef float pb_f32x4 __attribute__((ext_vector_type(4)));

// Each kind's round keeps only its own values live, so the loop holds
// nothing but the timed instructions and the loop counter.
template <int KIND>
__device__ __forceinline__ float issue_round(int iters, int lane, long long* t0, long long* t1, long long* r0,
                                             long long* r1) {
  if constexpr (KIND == 0) {
    pb_bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.01f * float(lane + i));
      b[i] = (__bf16)(0.02f * float(lane - i));
    }
    // distinct starting values keep the eight chains from being merged
    pb_f32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = pb_f32x4{float(lane + i), float(lane - i), float(lane * i), float(i - 2 * lane)};
    *r0 = __builtin_amdgcn_s_memrealtime();
    *t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
    }
    *t1 = __builtin_amdgcn_s_memtime();
    *r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
    return s;
  } else if constexpr (KIND == 2) {
    uint32_t u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = (uint32_t(lane * 16 + i) * 0x01010101u) & 0x3F3F3F3Fu;
    *r0 = __builtin_amdgcn_s_memrealtime();
    *t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const pb_bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[i], 1.0f, false);
        const pb_bf16x2 q = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u[i + 1], 1.0f, true);
        u[i] = __builtin_bit_cast(uint32_t, r);
        u[i + 1] = __builtin_bit_cast(uint32_t, q);
      }
    }
    *t1 = __builtin_amdgcn_s_memtime();
    *r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __uint_as_float(u[i] & 0x3F7FFFFFu);
    return s;
  } else {
    float f[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) f[i] = 0.001f * float(lane + i);
    // register operands (no literal), so the fma takes its 4-byte
    // accumulate form, as the decode's fp32 arithmetic mostly does
    const float m = 1e-7f * float(lane + 1);
    *r0 = __builtin_amdgcn_s_memrealtime();
    *t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 32; ++i) f[i] = KIND == 1 ? __builtin_fmaf(m, 0.5f, f[i]) : __builtin_amdgcn_exp2f(f[i]);
    }
    *t1 = __builtin_amdgcn_s_memtime();
    *r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += f[i];
    return s;
  }
}

// No launch bound: under a 256-thread bound the compiler rotates the MFMA
// accumulators between register ranges inside the loop, which adds moves.
template <int KIND>
__global__ void issue_kernel(int iters, long long* __restrict__ cycles, float* __restrict__ sink) {
  extern __shared__ int lds_hold[];
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) lds_hold[0] = iters;
  __syncthreads();
  long long t0, t1, r0, r1;
  float s;
  if constexpr (KIND == 4) {
    // waves 0-3 issue MFMAs, waves 4-7 (the SIMDs' second waves) fp32 fmas
    if (threadIdx.x < 256)
      s = issue_round<0>(iters, lane, &t0, &t1, &r0, &r1);
    else
      s = issue_round<1>(iters * 4, lane, &t0, &t1, &r0, &r1);
  } else {
    s = issue_round<KIND>(iters, lane, &t0, &t1, &r0, &r1);
  }
  s += float(lds_hold[0] & 1);
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
  // HW_ID (hardware register 4) bits 5:4 hold the wave's SIMD
  const int simd = __builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));
  if (lane == 0) {
    long long* c = cycles + (int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 3;
    c[0] = t1 - t0;
    c[1] = r1 - r0;
    c[2] = simd;
  }
}

// kind in [0, 5); waves_per_simd 1 or 2 (2 for kind 4) (workgroups of 256 or 512
// threads); `cycles`: device int64 [blocks * 4 * waves_per_simd * 3], per
// wave the s_memtime cycles, the s_memrealtime ticks (100 MHz) of the same
// interval and the wave's SIMD; `sink`: device float [blocks * 256 *
// waves_per_simd].  One workgroup per CU: 96 KiB of LDS each.
extern "C" int issue_rate_probe(int kind, int iters, int waves_per_simd, void* cycles, void* sink, int blocks,
                                void* stream) {
  if (!cycles || !sink || kind < 0 || kind > 4 || iters < 1 || blocks < 1 || waves_per_simd < 1 ||
      waves_per_simd > 2 || (kind == 4 && waves_per_simd != 2))
    return -1;
  const int threads = 256 * waves_per_simd;
  const size_t lds = 96 * 1024;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  long long* c = static_cast<long long*>(cycles);
  float* k = static_cast<float*>(sink);
#define ISSUE_CASE(K)                                                                                    \
  case K:                                                                                                \
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&issue_kernel<K>),                            \
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)         \
      return -2;                                                                                         \
    hipLaunchKernelGGL(issue_kernel<K>, dim3(blocks), dim3(threads), lds, s, iters, c, k);              \
    break;
  switch (kind) {
    ISSUE_CASE(0)
    ISSUE_CASE(1)
    ISSUE_CASE(2)
    ISSUE_CASE(3)
    ISSUE_CASE(4)
  }
#undef ISSUE_CASE
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
