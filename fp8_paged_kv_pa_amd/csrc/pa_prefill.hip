// Paged attention for long query segments (prompt-length q_len) over the
// page-shuffled e4m3fn cache (gfx950).
//
// It computes what the decode kernel computes -- row i of a q_len-L request
// sees context_len - L + i + 1 tokens (ROCm/ATOM pull request 2122, section
// 2), the per-token K scale multiplies each score and the per-token V scale
// each weight, scalar scales fold into the score scale and the normalized
// output (vllm-project/vllm pull request 52060, "Suggested Fix") -- for the
// per-token-as-decode prefill the pages run through the same contract
// (ROCm/ATOM pull request 2614, "Change"; the review of ROCm/ATOM pull
// request 2710, "Must fix" 1, sizes it at 16384 prompt tokens).  Only the
// kernel shape differs, because many rows share every page:
//
// A workgroup of 4 waves owns 8 consecutive query positions of one request
// and KV head (128 query rows); wave w owns positions 2w and 2w+1 (two
// 16-head row tiles, as a two-row decode wave).  The workgroup streams the
// 32-token chunks its last row sees, once: each of its 256 lanes loads 16
// bytes of K and 16 of V (the same bytes a decode wave's lane loads as its
// MFMA operands), converts them exactly to bf16 and stores them in LDS at
// the operand position; after a barrier every wave reads its operands from
// there.  So a chunk is fetched and converted once per 128 rows instead of
// once per 32, and the waves' LDS reads are 16 contiguous bytes per lane.
// The products, the online softmax (exp2 domain, the running max raised
// lazily), the P' = p * v_scale bf16 hi + lo pair and the output are those
// of the decode kernel.  Two chunks are in flight per lane in registers and
// LDS is double-buffered, one barrier per chunk.  Two workgroups share a CU
// (two waves per SIMD, from different workgroups, so their barriers do not
// line the two waves of a SIMD up).
//
// Long contexts with few rows split into partitions of pages whose (max,
// sum, accumulator) partials the decode's merge kernel combines; otherwise
// each workgroup writes its bf16 rows directly.  Workgroups go out
// heaviest first (the last query positions of a causal segment see the
// most tokens), so the dispatcher balances the CUs.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace fp8pa {

namespace {

constexpr int kPfPos = kPrefillPositions;  // query positions per workgroup
constexpr int kPfWaves = 4;
constexpr int kPfRing = 2;  // chunks in flight per lane beyond the one being staged
constexpr int kPfOcc = 2;   // workgroups per CU (two waves per SIMD)
constexpr int kPfRows = kPfPos / kPfWaves;  // query positions (16-head row tiles) per wave
static_assert(kPfRows * kPfWaves == kPfPos, "every wave owns the same number of positions");
constexpr float kPfLazy = 8.0f;  // log2 headroom before the running max moves

// One chunk (32 tokens of a (page, KV head) block) in LDS, as bf16 operands:
// K operand (token tile tt, k-step j) of lane l at k[4 tt + j][l], V
// operand of d-tile d at v[d][l], and the chunk's 32 K and V scales.
struct PfChunk {
  u32x4 k[8][kWave];
  u32x4 v[8][kWave];
  f32x4 ks[8];
  f32x4 vs[8];
};

// One lane's share of a chunk as loaded.  FP8: 16 bytes of K and of V
// (lane 64i + l holds row i of the chunk, the bytes decode lane l loads as
// its i-th piece) and, in waves 0 and 1, 16 bytes of the K or V scales.
// bf16 cache (8 rows of 1 KiB per chunk, each 16-byte piece one operand):
// rows i and i + 4 of K and of V.
template <bool BF>
struct PfLoad {
  u32x4 k[BF ? 2 : 1], v[BF ? 2 : 1];
  f32x4 s;
};

template <bool PER_TOKEN, bool BF>
__global__ __launch_bounds__(kWave * kPfWaves, kPfOcc) void pa_prefill_main(DecodeArgs a) {
  static_assert(!(BF && PER_TOKEN), "a bf16 cache carries no scales");
  __shared__ PfChunk sm[2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of each 16-token tile
  const int hr = lane & 15;  // query head within the GQA group
  const int Hq = 16 * a.hkv;

  // workgroup -> (row group gi, request b, KV head h, partition part), the
  // last row groups (most tokens) first
  const uint32_t per_group = uint32_t(a.batch) * uint32_t(a.hkv) * uint32_t(a.parts);
  const int gi = a.groups - 1 - int(blockIdx.x / per_group);
  uint32_t rem = blockIdx.x % per_group;
  const int part = int(rem % uint32_t(a.parts));
  rem /= uint32_t(a.parts);
  const int h = int(rem % uint32_t(a.hkv));
  const int b = int(rem / uint32_t(a.hkv));

  int start, L;
  if (a.cu_seqlens_q) {
    // clamped into [0, rows): a malformed cu can only give wrong values
    start = min(max(a.cu_seqlens_q[b], 0), a.rows);
    L = min(max(a.cu_seqlens_q[b + 1], start), a.rows) - start;
  } else {
    L = a.uniform_q_len;
    start = b * L;
  }
  const int i0 = gi * kPfPos;
  if (i0 >= L) return;  // the whole workgroup: no rows of this request here
  const int npos = min(kPfPos, L - i0);
  const int ctx = a.context_lens[b];
  const int cap = a.width * 128;
  // row i of the request sees tokens t < ctx - L + i + 1
  const int lim_group = max(0, min(ctx - L + i0 + npos, cap));  // the group's last row
  const int wp = kPfRows * wave;                                 // the wave's first position in the group
  const int nrows = max(0, min(kPfRows, npos - wp));
  const int lim0 = ctx - L + i0 + wp + 1;                        // the wave's first row
  const int lim_w0 = max(0, min(lim0, cap));
  const int lim_w1 = max(0, min(lim0 + max(nrows, 1) - 1, cap));
  const int row0 = start + i0 + min(wp, npos - 1);               // a real row for every wave

  // this partition's chunks of the group's tokens
  const int c0 = part * a.ppp * 4;
  const int c1 = (min((part + 1) * a.ppp * 128, lim_group) + 31) >> 5;

  float k_fold = a.sm_log2;  // scalar / none: the K scale folds into the score scale
  float v_fold = 1.0f;       // ... and the V scale into the normalized output
  if constexpr (!PER_TOKEN) {
    if (a.k_scale) k_fold *= *a.k_scale;
    if (a.v_scale) v_fold = *a.v_scale;
  }

  // query operands: B of S^T = K Q^T, lane = (head hr, dims 8g..8g+7 of
  // each 32-dim k-step); a wave with one row computes a copy in its second
  bf16x8 qop[kPfRows][4];
#pragma unroll
  for (int r = 0; r < kPfRows; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* qp = a.q + int64_t(row0 + min(r, max(nrows, 1) - 1)) * a.q_row_stride +
                           int64_t(16 * h + hr) * a.q_head_stride + 32 * j + 8 * g;
      qop[r][j] = *reinterpret_cast<const bf16x8*>(qp);
    }
  }

  f32x4 acc[kPfRows][8];
  float m_run[kPfRows], l_run[kPfRows];
#pragma unroll
  for (int r = 0; r < kPfRows; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[r][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- loads: lane 64i + l takes row i (1 KiB of 64 x 16 bytes) of the
  // chunk's K and V (bf16: rows i and i + 4); waves 0 and 1, lanes < 8, the
  // chunk's K or V scales
  constexpr int kBlk = BF ? 2 * kBlockBytes : kBlockBytes;  // one (page, head) block
  constexpr int kChunkBytes = kBlk / 4;                     // one 32-token chunk of it
  const int kv_off = 1024 * wave + 16 * lane;
  // (scalar loads, off the vector-memory counter of the K/V stream)
  const const_i32_ptr bt = as_const(a.block_table + int64_t(b) * a.bt_stride);
  auto issue = [&](int c, PfLoad<BF>& d) -> bool {
    const int n = c >> 2;
    const int P = (c < c1 && n < a.width) ? bt[n] : -1;
    const bool ok = P >= 0 && P < a.num_blocks;
    const int64_t blk = ok ? int64_t(P) * a.hkv + h : 0;
    const int nrec = ok ? kBlk : 0;
    const int off = (c & 3) * kChunkBytes + kv_off;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.k_cache + blk * kBlk, nrec);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.v_cache + blk * kBlk, nrec);
#pragma unroll
    for (int i = 0; i < (BF ? 2 : 1); ++i) {
      d.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 4096 * i, 0, 0);
      d.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off + 4096 * i, 0, 0);
    }
    if constexpr (PER_TOKEN) {
      // every lane issues it (so each step has the same loads in flight
      // and the waits before staging count exactly); only waves 0 and 1,
      // lanes < 8, are in range, the rest read past the 512-byte resource
      // and get zeros without a memory access
      const float* sp = (wave == 1 ? a.v_scale : a.k_scale) + blk * 128;
      const int soff = (wave < 2 && lane < 8) ? (c & 3) * 128 + 16 * lane : 512;
      d.s = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(block_rsrc(sp, ok ? 512 : 0), soff, 0, 0));
    }
    return ok;
  };
  // convert a loaded chunk into LDS buffer s; V bytes of tokens the group
  // does not see are zeroed (those slots may never have been written, and a
  // NaN there would survive a zero weight)
  auto stage = [&](const PfLoad<BF>& d, int c, PfChunk& s) {
    u32x4 v[BF ? 2 : 1];
#pragma unroll
    for (int i = 0; i < (BF ? 2 : 1); ++i) v[i] = d.v[i];
    const int t0 = 32 * c;
    if (t0 + 32 > lim_group) {
      keep_branch();
      if constexpr (BF) {
        // bf16 V row: word w holds the lane's slots 2w and 2w+1 of one dim
        // (slot e <-> token t0 + 16*(e/4) + 4g + e%4)
        uint32_t m[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          m[w] = 0;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int e = 2 * w + s2;
            if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) < lim_group) m[w] |= 0xFFFFu << (16 * s2);
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          v[i][0] &= m[0];
          v[i][1] &= m[1];
          v[i][2] &= m[2];
          v[i][3] &= m[3];
        }
      } else {
        uint32_t m0 = 0, m1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (t0 + 4 * g + e < lim_group) m0 |= 0xFFu << (8 * e);
          if (t0 + 16 + 4 * g + e < lim_group) m1 |= 0xFFu << (8 * e);
        }
        v[0][0] &= m0;
        v[0][1] &= m1;
        v[0][2] &= m0;
        v[0][3] &= m1;
      }
    }
    if constexpr (BF) {
      // row r of a bf16 chunk is K operand r (token tile r/4, k-step r%4)
      // and V operand (d-tile) r, as loaded
      s.k[wave][lane] = d.k[0];
      s.k[wave + 4][lane] = d.k[1];
      s.v[wave][lane] = v[0];
      s.v[wave + 4][lane] = v[1];
    } else {
      // K row i: token tile i/2, k-steps 2(i%2) and 2(i%2)+1; V row i: d-tiles 2i, 2i+1
      const int kj = 4 * (wave >> 1) + 2 * (wave & 1);
      s.k[kj][lane] = __builtin_bit_cast(u32x4, fp8x8_to_bf16x8(d.k[0][0], d.k[0][1]));
      s.k[kj + 1][lane] = __builtin_bit_cast(u32x4, fp8x8_to_bf16x8(d.k[0][2], d.k[0][3]));
      s.v[2 * wave][lane] = __builtin_bit_cast(u32x4, fp8x8_to_bf16x8(v[0][0], v[0][1]));
      s.v[2 * wave + 1][lane] = __builtin_bit_cast(u32x4, fp8x8_to_bf16x8(v[0][2], v[0][3]));
    }
    if constexpr (PER_TOKEN) {
      if (wave == 0 && lane < 8) s.ks[lane] = d.s * k_fold;
      if (wave == 1 && lane < 8) s.vs[lane] = d.s;
    }
  };

  // ---- one chunk of this wave's two rows ----------------------------------
  auto process = [&](const PfChunk& s, int c, bool ok) {
    const int t0 = 32 * c;
    // this wave's rows see none of it, or its page is outside the cache (a
    // table entry out of range: the chunk is skipped, as the decode does)
    if (nrows == 0 || t0 >= lim_w1 || !ok) return;
    const bool full = t0 + 32 <= lim_w0;
    // per-token factors of this lane's 8 tokens (slot e <-> token
    // t0 + 16*(e/4) + 4g + e%4): K scale folded with sm*log2(e) (folded when
    // staged), V scale
    float kc[8], vsf[8];
    if constexpr (PER_TOKEN) {
      const f32x4 ka = s.ks[g], kb = s.ks[4 + g], va = s.vs[g], vb = s.vs[4 + g];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kc[e] = ka[e];
        kc[4 + e] = kb[e];
        vsf[e] = va[e];
        vsf[4 + e] = vb[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kc[e] = k_fold;
        vsf[e] = 1.0f;
      }
    }
    f32x4 st[kPfRows][2];
#pragma unroll
    for (int r = 0; r < kPfRows; ++r) st[r][0] = st[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 k0 = __builtin_bit_cast(bf16x8, s.k[j][lane]);
      const bf16x8 k1 = __builtin_bit_cast(bf16x8, s.k[4 + j][lane]);
#pragma unroll
      for (int r = 0; r < kPfRows; ++r) {
        st[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[r][j], st[r][0], 0, 0, 0);
        st[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[r][j], st[r][1], 0, 0, 0);
      }
    }

    // online softmax per row; P' = p * v_scale as a bf16 hi + lo pair (hi
    // the top 8 significant bits by truncation, lo = P' - hi exact in fp32)
    bf16x8 phi[kPfRows], plo[kPfRows];
#pragma unroll
    for (int r = 0; r < kPfRows; ++r) {
      const float mu = (m_run[r] == -INFINITY) ? 0.0f : m_run[r];
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = fmaf(st[r][0][e], kc[e], -mu);
        x[4 + e] = fmaf(st[r][1][e], kc[4 + e], -mu);
      }
      const int lim_r = max(0, min(lim0 + min(r, max(nrows, 1) - 1), cap));
      if (!full) {
        keep_branch();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = t0 + 16 * (e >> 2) + 4 * g + (e & 3);
          x[e] = t < lim_r ? x[e] : -INFINITY;
        }
      }
      const float lm = max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), max2f(x[6], x[7]));
      const bool need = lm > (m_run[r] == -INFINITY ? -INFINITY : kPfLazy);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        float gm = fmaxf(lm, __shfl_xor(lm, 16, kWave));
        gm = fmaxf(gm, __shfl_xor(gm, 32, kWave));
        const float mn = fmaxf(m_run[r], gm + mu);
        const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - mn);
        l_run[r] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[r][d] *= alpha;
        m_run[r] = mn;
        const float shift = (mn == -INFINITY) ? 0.0f : mn - mu;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] -= shift;
      }
      float pe[8], pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = __builtin_amdgcn_exp2f(x[e]);
        pv[e] = pe[e] * vsf[e];
      }
      if (PER_TOKEN && !full) {
        // a token past this row's cutoff but seen by a later row of the
        // group has a scale that need not be finite for this row's zero
        keep_branch();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = t0 + 16 * (e >> 2) + 4 * g + (e & 3);
          pv[e] = t < lim_r ? pv[e] : 0.0f;
        }
      }
      uint32_t hb[8];
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hb[e] = __float_as_uint(pv[e]) & 0xFFFF0000u;
        lo[e] = pv[e] - __uint_as_float(hb[e]);
      }
      l_run[r] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
      u32x4 hw;
#pragma unroll
      for (int e = 0; e < 4; ++e) hw[e] = __builtin_amdgcn_perm(hb[2 * e + 1], hb[2 * e], 0x07060302u);
      phi[r] = __builtin_bit_cast(bf16x8, hw);
#pragma unroll
      for (int e = 0; e < 8; ++e) plo[r][e] = (__bf16)lo[e];
    }

    // O^T += V^T P'^T
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const bf16x8 vop = __builtin_bit_cast(bf16x8, s.v[d][lane]);
#pragma unroll
      for (int r = 0; r < kPfRows; ++r) {
        acc[r][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi[r], acc[r][d], 0, 0, 0);
        acc[r][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo[r], acc[r][d], 0, 0, 0);
      }
    }
  };

  // ---- stream the chunks: chunk c in LDS buffer (c - c0) % 2 while the
  // loads of c + 1 and c + 2 are in flight in the register ring ------------
  if (c0 < c1) {
    PfLoad<BF> first, ring[kPfRing];
    bool ok_ring[kPfRing], ok_buf[2];
    ok_buf[0] = issue(c0, first);
#pragma unroll
    for (int k = 0; k < kPfRing; ++k) ok_ring[k] = issue(c0 + 1 + k, ring[k]);
    stage(first, c0, sm[0]);
    __syncthreads();
    for (int c = c0; c < c1; c += 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int cc = c + k;
        const int q = k % kPfRing;  // ring slot holding chunk cc + 1
        if (cc < c1) process(sm[k], cc, ok_buf[k]);
        // Staging and loads run on every step, also past the range (those
        // loads cover 0 bytes and return zeros; that staging lands in a
        // buffer nothing reads again), so every step has the same loads in
        // flight and the wait before each staging counts exactly the newer
        // step's loads instead of draining all of them.
        stage(ring[q], cc + 1, sm[k ^ 1]);
        ok_buf[k ^ 1] = ok_ring[q];
        ok_ring[q] = issue(cc + 1 + kPfRing, ring[q]);
        __syncthreads();
      }
    }
  }

  // ---- this wave's rows: bf16 output, or the partition's partial ---------
#pragma unroll
  for (int r = 0; r < kPfRows; ++r) {
    if (r >= nrows) break;
    float lh = l_run[r];
    lh += __shfl_xor(lh, 16, kWave);  // the head's four lane groups hold its tokens' sums
    lh += __shfl_xor(lh, 32, kWave);
    const int row = start + i0 + wp + r;
    const int qh = 16 * h + hr;
    if (a.parts == 1) {
      const float inv = lh > 0.0f ? v_fold / lh : 0.0f;
      uint16_t* op = a.out + int64_t(row) * a.out_row_stride + int64_t(qh) * a.out_head_stride + 4 * g;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t w0 = uint32_t(f32_to_bf16_rne(acc[r][d][0] * inv)) |
                            (uint32_t(f32_to_bf16_rne(acc[r][d][1] * inv)) << 16);
        const uint32_t w1 = uint32_t(f32_to_bf16_rne(acc[r][d][2] * inv)) |
                            (uint32_t(f32_to_bf16_rne(acc[r][d][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(op + 16 * d) = uint2{w0, w1};
      }
    } else {
      const int64_t pi = (int64_t(part) * a.rows + row) * Hq + qh;
      float* ap = a.part_acc + pi * 128 + 4 * g;
#pragma unroll
      for (int d = 0; d < 8; ++d) *reinterpret_cast<f32x4*>(ap + 16 * d) = acc[r][d];
      if (g == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * pi) = float2{m_run[r], lh};
    }
  }
}

}  // namespace

hipError_t launch_prefill_main(const DecodeArgs& a, int64_t grid, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
  const dim3 block(kWave * kPfWaves);
  auto go = [&](auto kernel) {
    if (e0 || e1) hipExtLaunchKernelGGL(kernel, dim3(uint32_t(grid)), block, 0, s, e0, e1, 0, a);
    else hipLaunchKernelGGL(kernel, dim3(uint32_t(grid)), block, 0, s, a);
  };
  if (a.kv_bf16) go(pa_prefill_main<false, true>);
  else if (a.scale_mode == PA_SCALE_PER_TOKEN) go(pa_prefill_main<true, false>);
  else go(pa_prefill_main<false, false>);
  return hipGetLastError();
}

}  // namespace fp8pa
