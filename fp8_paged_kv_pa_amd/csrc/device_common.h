// Device-side helpers for gfx950: vector types, FP8 <-> bf16/f32
// conversion, wave reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fp8pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Eight OCP e4m3fn bytes (two dwords, byte 0 first) to eight bf16.  Every
// e4m3fn value, subnormals included, is a bf16 value, so this is exact.
// v_cvt_scalef32_pk_bf16_fp8 converts the two bytes of the selected 16-bit
// half; a scale of 1.0 leaves the values unchanged.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// fp32 -> e4m3fn byte: round to nearest, ties to even, saturate to +-448
// (infinities included); NaN -> 0x7F with the sign.  Pure integer work on
// the fp32 bit pattern, so its result does not depend on any conversion
// instruction's overflow mode.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448
  if (a < 0x3C800000u) {                       // |y| < 2^-6: spacing 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scale, RNE
    return sign | uint32_t(m);                 // 8 -> 0x08 = 2^-6, the smallest normal
  }
  // normal: biased e4m3 exponent = fp32 exponent - 120, three mantissa bits
  uint32_t code = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1;  // carry may bump exponent
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// Cross-lane max / sum of a wave without LDS: DPP within rows of 16 lanes
// (swap neighbours, swap pairs, rotate by 4, rotate by 8 -- every lane of a
// row then holds the row's result), then the four rows through readlane.
// Every lane gets the result.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  int b = __builtin_bit_cast(int, v);
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
  b = __builtin_bit_cast(int, v);
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
  b = __builtin_bit_cast(int, v);
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x124, 0xF, 0xF, false)));  // row_ror 4
  b = __builtin_bit_cast(int, v);
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x128, 0xF, 0xF, false)));  // row_ror 8
  b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ float wave_max(float v) { return wave_reduce<true>(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<false>(v); }

// Unsigned add / max / min over a wave without LDS: DPP within rows of 16
// lanes (swap neighbours, swap pairs, rotate by 4, rotate by 8), then the
// four rows through readlane.  Every lane gets the result.
enum class UOp { ADD, MAX, MIN };
template <UOp OP>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto op = [](uint32_t x, uint32_t y) { return OP == UOp::ADD ? x + y : (OP == UOp::MAX ? max(x, y) : min(x, y)); };
  int b = int(v);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
  b = int(v);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
  b = int(v);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(b, b, 0x124, 0xF, 0xF, false)));  // row_ror 4
  b = int(v);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(b, b, 0x128, 0xF, 0xF, false)));  // row_ror 8
  b = int(v);
  return op(op(uint32_t(__builtin_amdgcn_readlane(b, 0)), uint32_t(__builtin_amdgcn_readlane(b, 16))),
            op(uint32_t(__builtin_amdgcn_readlane(b, 32)), uint32_t(__builtin_amdgcn_readlane(b, 48))));
}

// Inclusive prefix sum over a wave by DPP: within rows of 16 lanes (add
// the lane 1, 2, 4, 8 below; lanes with no such lane in the row add 0),
// then across rows (lane 15 of rows 0 and 2 into rows 1 and 3, then lane
// 31 into rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr 1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr 2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr 4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr 8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast 15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast 31
  return x;
}

// An empty volatile asm: a block that holds one cannot be speculated, so
// the compiler keeps a uniform branch around the tail-chunk masks instead of
// turning them into selects that every full chunk would execute.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Maxima of a chunk's scores in 4 instructions for 8 values.  fmaxf lowers
// to maxnum, for which the compiler first quiets each input with a v_max of
// the value with itself; the scores are products and selects, never
// signaling NaNs, so v_max3 / v_max take them as they are (a quiet NaN
// yields the other operand either way).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Word 3 of a gfx9 buffer resource: raw (untyped) 32-bit data format, no
// swizzle, no per-lane index stride.
constexpr int kRsrcWord3 = 0x00020000;

// A raw buffer over `bytes` bytes at `p` (0: every access is out of range,
// which returns zeros without touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), short(0), bytes, kRsrcWord3);
}

// Read-only tables (block table, sparse lists) read through the constant
// address space: uniform reads become scalar loads, counted apart from the
// vector loads of the KV stream, so waiting for a table entry never waits
// for KV bytes in flight.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
__device__ __forceinline__ const_i32_ptr as_const(const int32_t* p) { return (const_i32_ptr)(p); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

}  // namespace fp8pa
