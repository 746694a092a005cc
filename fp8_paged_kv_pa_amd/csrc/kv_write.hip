// kv_quant_write: quantize new K/V rows to e4m3fn and store them in the
// page-shuffled cache, with per-token amax/448 scales (or a scalar scale,
// or none).  One wavefront per (token, KV head); each lane owns dims
// 2*lane and 2*lane+1.
//
// Per-token scale = fl32(amax / 448) and code = RNE-satfinite(fl32(x/scale))
// follow the definition of the per-token/head FP8 cache in ROCm/ATOM pull
// request 2614 ("Problem": page-shuffled FP8 with per-token K/V scales) and
// the scale modes of vllm-project/vllm pull request 52060 ("Suggested
// Fix").  It is the only cache writer of the library (ROCm/ATOM pull request
// 2710 review, "Smaller": one shared writer so the FP8 and non-FP8 branches
// cannot drift), so the unquantized bf16 cache is written here too.
#include "device_common.h"
#include "launch.h"

namespace fp8pa {

namespace {

constexpr int kWriteWaves = 4;

__device__ __forceinline__ void load_pair(const void* base, int64_t off, int bf16, float* x0,
                                          float* x1) {
  if (bf16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const uint16_t*>(base) + off);
    *x0 = __uint_as_float(w << 16);
    *x1 = __uint_as_float(w & 0xFFFF0000u);
  } else {
    const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + off);
    *x0 = v.x;
    *x1 = v.y;
  }
}

// Quantize this lane's two values of one 128-wide row.  Returns the two
// codes (low byte = even dim) and, through *scale_out, the stored scale.
__device__ __forceinline__ uint32_t quantize_pair(float x0, float x1, int mode, const float* scalar,
                                                  float* scale_out) {
  float s = 1.0f;
  bool divide = false;
  if (mode == PA_SCALE_PER_TOKEN) {
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    s = amax / 448.0f;  // IEEE fp32 division
    divide = s != 0.0f;
  } else if (mode == PA_SCALE_SCALAR) {
    s = *scalar;
    divide = true;
  }
  float y0 = x0, y1 = x1;
  if (divide) {
    y0 = x0 / s;
    y1 = x1 / s;
  }
  *scale_out = s;
  return f32_to_e4m3(y0) | (f32_to_e4m3(y1) << 8);
}

// fp32 -> bf16 bits: round to nearest, ties to even, on the 16 dropped
// bits; NaN stays NaN (quiet bit set, sign kept).  Integer work, so the
// stored bits do not depend on a conversion instruction's NaN handling.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The unquantized cache: bf16 elements in the bf16 page layout (same
// chunking as the FP8 pages, 8 elements per 16-byte lane operand).
__device__ __forceinline__ void store_bf16(const WriteArgs& a, int64_t page, int h, int o, int lane,
                                           float k0, float k1, float v0, float v1) {
  const int64_t blk = (page * a.hkv + h) * int64_t(16384);
  uint16_t* kc = reinterpret_cast<uint16_t*>(a.k_cache) + blk;
  uint16_t* vc = reinterpret_cast<uint16_t*>(a.v_cache) + blk;
  const int c = o >> 5, tau = (o >> 4) & 1;
  // K: dims 2*lane and 2*lane+1 are adjacent elements (u even, u+1)
  {
    const int d = 2 * lane;
    const int j = d >> 5, g = (d >> 3) & 3, u = d & 7, r = o & 15;
    const int off = 4096 * c + 512 * (4 * tau + j) + 8 * (16 * g + r) + u;
    *reinterpret_cast<uint32_t*>(kc + off) = f32_to_bf16_bits(k0) | (f32_to_bf16_bits(k1) << 16);
  }
  // V: the two dims sit in pieces 8 elements apart
  {
    const int w = o & 15, g = w >> 2, e = 4 * tau + (w & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int d = 2 * lane + s;
      const int delta = d >> 4, r = d & 15;
      const int off = 4096 * c + 512 * delta + 8 * (16 * g + r) + e;
      vc[off] = uint16_t(f32_to_bf16_bits(s ? v1 : v0));
    }
  }
}

__global__ __launch_bounds__(kWave * kWriteWaves) void kv_write_kernel(WriteArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = int64_t(blockIdx.x) * kWriteWaves + (threadIdx.x >> 6);
  if (pair >= a.tokens * a.hkv) return;  // whole wave exits together
  const int64_t t = pair / a.hkv;
  const int h = int(pair - t * a.hkv);
  // inputs and slot in one round trip: the value loads do not depend on the slot
  float k0, k1, v0, v1;
  load_pair(a.k_new, t * a.k_tok_stride + h * a.k_head_stride + 2 * lane, a.in_bf16, &k0, &k1);
  load_pair(a.v_new, t * a.v_tok_stride + h * a.v_head_stride + 2 * lane, a.in_bf16, &v0, &v1);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * 128) return;
  const int64_t page = slot >> 7;
  const int o = int(slot & 127);
  if (a.out_bf16) {
    store_bf16(a, page, h, o, lane, k0, k1, v0, v1);
    return;
  }

  float ks, vs;
  const uint32_t kc = quantize_pair(k0, k1, a.scale_mode, a.k_scale, &ks);
  const uint32_t vc = quantize_pair(v0, v1, a.scale_mode, a.v_scale, &vs);

  const int64_t blk = (page * a.hkv + h) * int64_t(16384);
  const int c = o >> 5, tau = (o >> 4) & 1;

  // K: dims d = 2*lane, 2*lane+1 share one 8-byte run (u even, u+1).
  {
    const int d = 2 * lane;
    const int j = d >> 5, g = (d >> 3) & 3, u = d & 7, r = o & 15;
    const int off = 4096 * c + 1024 * (2 * tau + (j >> 1)) + 16 * (16 * g + r) + 8 * (j & 1) + u;
    *reinterpret_cast<uint16_t*>(a.k_cache + blk + off) = uint16_t(kc);
  }
  // V: each dim goes to a different 16-byte piece.
  {
    const int w = o & 15, g = w >> 2, e = 4 * tau + (w & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int d = 2 * lane + s;
      const int delta = d >> 4, r = d & 15;
      const int off = 4096 * c + 1024 * (delta >> 1) + 16 * (16 * g + r) + 8 * (delta & 1) + e;
      a.v_cache[blk + off] = uint8_t(vc >> (8 * s));
    }
  }
  if (a.scale_mode == PA_SCALE_PER_TOKEN && lane == 0) {
    const int64_t si = (page * a.hkv + h) * 128 + o;
    a.k_scale[si] = ks;
    a.v_scale[si] = vs;
  }
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, hipStream_t stream) {
  const int64_t pairs = a.tokens * a.hkv;
  if (pairs == 0) return hipSuccess;
  const int64_t grid = (pairs + kWriteWaves - 1) / kWriteWaves;
  hipLaunchKernelGGL(kv_write_kernel, dim3(uint32_t(grid)), dim3(kWave * kWriteWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp8pa
