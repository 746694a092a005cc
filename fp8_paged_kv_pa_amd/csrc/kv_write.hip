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
// cannot drift), so the unquantized bf16 cache is written here too.  Its
// per-token load, quantization and FP8 and bf16 stores live in
// writer_common.h, which the decode kernel's fused write (pa_decode_write)
// calls as well.
//
// The fused variant (kv_norm_rope_write) applies the key's RMS norm and
// rotary embedding to K in registers before the same quantize-and-store
// code, and transforms the query alongside in the same launch (ROCm/ATOM
// pull request 2710, "Changes": query/key norm, rotary embedding and cache
// write fused; its review, "Smaller": the norm-then-rope path and the
// rope-only path must share one cache-write branch).  Every fp32 step is a
// single IEEE operation rounded to nearest even, with no fused
// multiply-add, in a fixed order (see transform_pair), so the codes and
// scales it writes are reproducible bit for bit.
#include "device_common.h"
#include "launch.h"
#include "writer_common.h"

namespace fp8pa {

namespace {

constexpr int kWriteWaves = 4;

// Sum over the wave of one value per lane as a balanced binary tree in lane
// order: at step k every lane adds the lane k apart (xor), so each partial is
// the sum of an aligned block of lanes and every lane ends with the same
// result, whatever the order of the two operands of each addition.
__device__ __forceinline__ float wave_tree_sum(float v) {
#pragma unroll
  for (int k = 1; k < kWave; k <<= 1) v += __shfl_xor(v, k, kWave);
  return v;
}

// RMS norm (with `w`) and rotary embedding of one 128-wide head row, of
// which this lane holds dims 2*lane and 2*lane+1 in x0, x1.  The fp32 order:
//   sq = x*x per dim; S = balanced binary tree over the dims in order
//   (x0^2 + x1^2 in the lane, then wave_tree_sum); m = S * 2^-7 (exact);
//   inv = 1 / sqrt(m + eps); y = (x * inv) * (offset + w);
//   a rotary pair (a, b) with table entries (c, s) becomes
//   (a*c - b*s, b*c + a*s).
// Each operation is one IEEE fp32 operation (division and square root
// correctly rounded), rounded to nearest even, never fused.
__device__ __forceinline__ void transform_pair(float& x0, float& x1, const float* w, const NormRopeArgs& n,
                                               int64_t pos, int lane) {
#pragma clang fp contract(off)
  if (w) {
    float sq = x0 * x0 + x1 * x1;
    const float S = wave_tree_sum(sq);
    const float m = S * 0.0078125f;
    const float v = m + n.eps;
    const float r = __builtin_sqrtf(v);
    const float inv = 1.0f / r;
    const float w0 = n.offset + w[2 * lane];
    const float w1 = n.offset + w[2 * lane + 1];
    x0 = (x0 * inv) * w0;
    x1 = (x1 * inv) * w1;
  }
  if (n.rot == 0) return;
  const float* cr = n.cos + pos * n.cos_stride;
  const float* sr = n.sin + pos * n.sin_stride;
  const int d = 2 * lane;
  if (n.neox) {
    // pairs (i, i + half); half is even, so a lane's two dims sit in one
    // half and their partners in one lane, half/2 lanes away
    const int half = n.rot >> 1;
    const bool first = d < half;
    const int partner = first ? lane + (half >> 1) : lane - (half >> 1);
    const float p0 = __shfl(x0, partner & (kWave - 1), kWave);
    const float p1 = __shfl(x1, partner & (kWave - 1), kWave);
    if (d < n.rot) {
      const int i = first ? d : d - half;
      const float c0 = cr[i], c1 = cr[i + 1], s0 = sr[i], s1 = sr[i + 1];
      if (first) {  // own = a, partner = b: a*c - b*s
        const float a0c = x0 * c0, b0s = p0 * s0, a1c = x1 * c1, b1s = p1 * s1;
        x0 = a0c - b0s;
        x1 = a1c - b1s;
      } else {      // own = b, partner = a: b*c + a*s
        const float b0c = x0 * c0, a0s = p0 * s0, b1c = x1 * c1, a1s = p1 * s1;
        x0 = b0c + a0s;
        x1 = b1c + a1s;
      }
    }
  } else if (d < n.rot) {
    // pairs (2i, 2i + 1): this lane's own two dims, table column i = lane
    const float c = cr[lane], s = sr[lane];
    const float ac = x0 * c, bs = x1 * s, bc = x1 * c, as = x0 * s;
    x0 = ac - bs;
    x1 = bc + as;
  }
}

// One query head of the fused writer: norm (its own weight) and rotary
// embedding, stored as bf16.
__device__ __forceinline__ void query_wave(const WriteArgs& a, int64_t qi, int lane) {
  const NormRopeArgs& n = a.nr;
  const int64_t t = qi / n.hq;
  const int h = int(qi - t * n.hq);
  float x0, x1;
  load_pair(n.q_in, t * n.q_tok_stride + h * n.q_head_stride + 2 * lane, n.q_bf16, &x0, &x1);
  const int64_t pos = min(max(n.positions[t], int64_t(0)), n.max_pos - 1);
  transform_pair(x0, x1, n.q_weight, n, pos, lane);
  uint16_t* op = n.q_out + t * n.qo_tok_stride + h * n.qo_head_stride + 2 * lane;
  *reinterpret_cast<uint32_t*>(op) = f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16);
}

template <bool NR>
__global__ __launch_bounds__(kWave * kWriteWaves) void kv_write_kernel(WriteArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = int64_t(blockIdx.x) * kWriteWaves + (threadIdx.x >> 6);
  const int64_t kv_pairs = a.tokens * a.hkv;
  if constexpr (NR) {
    // waves past the (token, KV head) pairs transform the query heads
    if (pair >= kv_pairs) {
      if (a.nr.q_in && pair < kv_pairs + a.tokens * a.nr.hq) query_wave(a, pair - kv_pairs, lane);
      return;  // whole wave exits together
    }
  }
  if (pair >= kv_pairs) return;  // whole wave exits together
  const int64_t t = pair / a.hkv;
  const int h = int(pair - t * a.hkv);
  // inputs and slot in one round trip: the value loads do not depend on the slot
  float k0, k1, v0, v1;
  load_pair(a.k_new, t * a.k_tok_stride + h * a.k_head_stride + 2 * lane, a.in_bf16, &k0, &k1);
  load_pair(a.v_new, t * a.v_tok_stride + h * a.v_head_stride + 2 * lane, a.in_bf16, &v0, &v1);
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_blocks * 128) return;  // the slot is the wave's: uniform
  if constexpr (NR) {
    const int64_t pos = min(max(a.nr.positions[t], int64_t(0)), a.nr.max_pos - 1);
    transform_pair(k0, k1, a.nr.k_weight, a.nr, pos, lane);
  }
  if (a.out_bf16) {
    store_token_bf16(a.k_cache, a.v_cache, a.hkv, slot, h, lane, f32_to_bf16_bits(k0) | (f32_to_bf16_bits(k1) << 16),
                     f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16));
    return;
  }

  float ks, vs;
  const uint32_t kc = quantize_pair(k0, k1, a.scale_mode, a.k_scale, &ks);
  const uint32_t vc = quantize_pair(v0, v1, a.scale_mode, a.v_scale, &vs);

  store_token_fp8(a.k_cache, a.v_cache, a.k_scale, a.v_scale, a.hkv, a.scale_mode, slot, h, lane, kc, vc, ks, vs);
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, hipStream_t stream) {
  int64_t pairs = a.tokens * a.hkv;
  if (a.nr.on && a.nr.q_in) pairs += a.tokens * a.nr.hq;
  if (pairs == 0) return hipSuccess;
  const int64_t grid = (pairs + kWriteWaves - 1) / kWriteWaves;
  if (a.nr.on)
    hipLaunchKernelGGL(kv_write_kernel<true>, dim3(uint32_t(grid)), dim3(kWave * kWriteWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_write_kernel<false>, dim3(uint32_t(grid)), dim3(kWave * kWriteWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp8pa
