// The cache writer's per-token steps, shared by the writer kernel
// (kv_write.hip) and the decode kernel's fused write of a step's new tokens
// (pa_decode.hip), so the two cannot drift (ROCm/ATOM pull request 2710
// review, "Smaller": one shared cache-write branch).  Internal to the
// library.
//
// A token row of 128 values is held by one wavefront, lane l owning dims 2l
// and 2l+1.  Per-token scale = fl32(amax / 448), code = RNE-satfinite of
// fl32(x / scale) (ROCm/ATOM pull request 2614, "Problem": page-shuffled FP8
// with per-token K/V scales; vllm-project/vllm pull request 52060,
// "Suggested Fix": the scalar and no-scale modes).
#pragma once

#include "../../include/fp8pa.h"
#include "device_common.h"

namespace fp8pa {

// Two adjacent input values (f32 or bf16) at element offset `off`.
__device__ __forceinline__ void load_pair(const void* base, int64_t off, int bf16, float* x0, float* x1) {
  if (bf16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + off);
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
// `scalar` is the caller's scale in SCALAR mode (unused otherwise).
__device__ __forceinline__ uint32_t quantize_pair_v(float x0, float x1, int mode, float scalar, float* scale_out) {
  float s = 1.0f;
  bool divide = false;
  if (mode == PA_SCALE_PER_TOKEN) {
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    s = amax / 448.0f;  // IEEE fp32 division
    divide = s != 0.0f;
  } else if (mode == PA_SCALE_SCALAR) {
    s = scalar;
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

// The same, reading the SCALAR-mode scale from `scalar`.
__device__ __forceinline__ uint32_t quantize_pair(float x0, float x1, int mode, const float* scalar,
                                                  float* scale_out) {
  return quantize_pair_v(x0, x1, mode, mode == PA_SCALE_SCALAR ? *scalar : 1.0f, scale_out);
}

// Stores this lane's two codes of token slot `slot` (page slot >> 7, offset
// slot & 127) for KV head h in the page-shuffled FP8 layout, and (lane 0)
// the token's per-token scales.  K: the two dims share one 8-byte run; V:
// each dim goes to a different 16-byte piece.
__device__ __forceinline__ void store_token_fp8(uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                                                int hkv, int mode, int64_t slot, int h, int lane, uint32_t kc,
                                                uint32_t vc, float ks, float vs) {
  const int64_t page = slot >> 7;
  const int o = int(slot & 127);
  const int64_t blk = (page * hkv + h) * int64_t(16384);
  const int c = o >> 5, tau = (o >> 4) & 1;
  {
    const int d = 2 * lane;
    const int j = d >> 5, g = (d >> 3) & 3, u = d & 7, r = o & 15;
    const int off = 4096 * c + 1024 * (2 * tau + (j >> 1)) + 16 * (16 * g + r) + 8 * (j & 1) + u;
    *reinterpret_cast<uint16_t*>(k_cache + blk + off) = uint16_t(kc);
  }
  {
    const int w = o & 15, g = w >> 2, e = 4 * tau + (w & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int d = 2 * lane + s;
      const int delta = d >> 4, r = d & 15;
      const int off = 4096 * c + 1024 * (delta >> 1) + 16 * (16 * g + r) + 8 * (delta & 1) + e;
      v_cache[blk + off] = uint8_t(vc >> (8 * s));
    }
  }
  if (mode == PA_SCALE_PER_TOKEN && lane == 0) {
    const int64_t si = (page * hkv + h) * 128 + o;
    k_scale[si] = ks;
    v_scale[si] = vs;
  }
}

// fp32 -> bf16 bits: round to nearest, ties to even, on the 16 dropped
// bits; NaN stays NaN (quiet bit set, sign kept).  Integer work, so the
// stored bits do not depend on a conversion instruction's NaN handling.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The unquantized cache: stores this lane's two K and two V elements
// (kb, vb: bf16 bits, low half = even dim) of token slot `slot` for KV
// head h in the bf16 page layout (the FP8 pages' chunking, 8 elements per
// 16-byte operand piece).  K: the two dims are adjacent elements; V: they
// sit in pieces 8 elements apart.
__device__ __forceinline__ void store_token_bf16(uint8_t* k_cache, uint8_t* v_cache, int hkv, int64_t slot, int h,
                                                 int lane, uint32_t kb, uint32_t vb) {
  const int64_t page = slot >> 7;
  const int o = int(slot & 127);
  const int64_t blk = (page * hkv + h) * int64_t(16384);
  uint16_t* kc = reinterpret_cast<uint16_t*>(k_cache) + blk;
  uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache) + blk;
  const int c = o >> 5, tau = (o >> 4) & 1;
  {
    const int d = 2 * lane;
    const int j = d >> 5, g = (d >> 3) & 3, u = d & 7, r = o & 15;
    const int off = 4096 * c + 512 * (4 * tau + j) + 8 * (16 * g + r) + u;
    *reinterpret_cast<uint32_t*>(kc + off) = kb;
  }
  {
    const int w = o & 15, g = w >> 2, e = 4 * tau + (w & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int d = 2 * lane + s;
      const int delta = d >> 4, r = d & 15;
      const int off = 4096 * c + 512 * delta + 8 * (16 * g + r) + e;
      vc[off] = uint16_t(vb >> (16 * s));
    }
  }
}

}  // namespace fp8pa
