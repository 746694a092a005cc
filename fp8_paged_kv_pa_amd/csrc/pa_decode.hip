// Paged decode attention over the page-shuffled e4m3fn cache (gfx950).
//
// What is computed (ROCm/ATOM pull request 2614, "Change": dense and sparse
// decode through one shuffled paged-decode contract with per-token FP8
// scales; ROCm/ATOM pull request 2122, section 2: row i of a q_len-L request
// sees context_len - L + i + 1 tokens; vllm-project/vllm pull request 52060,
// "Suggested Fix": scalar scales fold into the score scale and the
// normalized output):
//   out[row, 16h+j] = sum_t softmax_t(sm * <q, ks_t k_t>) * vs_t v_t
// over the row's tokens, exact softmax, split into partitions whose
// (max, sum, accumulator) partials a log-sum-exp merge combines (ROCm/ATOM
// pull request 2710 review, "Must fix" 1, names that partial scratch).
//
// Kernel shape.  A workgroup of 4 wavefronts owns (request or row, KV head,
// row group, partition).  Wave w handles token chunk w (32 tokens) of every
// page of the partition, so the 4 waves stream one page together.  Each
// lane's 16-byte loads are, byte for byte, its matrix-core operands (the
// cache layout is defined that way), so nothing goes through LDS in the
// loop:
//   S^T[token, head] = K[token, d] * Q^T[d, head]     (bf16 MFMA 16x16x32)
//   O^T[d, head]    += V^T[d, token] * P^T[token, head]
// Computing S transposed leaves each lane with one head and 8 tokens, which
// is exactly the B-operand of the P*V product: no transpose of P.  The
// e4m3 -> bf16 conversion is exact; the per-token K scale multiplies each
// score column once and the per-token V scale multiplies P, so no scale
// touches a 128-wide vector.  P' enters the P*V product as a bf16 hi + lo
// pair (two MFMAs), so its rounding stays near 2^-16 instead of bf16's 2^-9.
// Online softmax in the exp2 domain; the running max is only raised when a
// chunk exceeds it by more than 2^8, so P stays <= 256 and the rescale of
// the accumulators is rare.  The four waves' partials merge through LDS at
// the end; with one partition the workgroup writes bf16 output directly.
//
// The unquantized bf16 cache (the control the FP8 cache is measured
// against) runs the same kernel: its pages keep the same chunking with
// 2-byte elements, so each 16-byte load is one bf16 operand as is.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "writer_common.h"
#include "launch.h"

namespace fp8pa {

namespace {


constexpr float kLazyMax = 8.0f;  // log2 headroom before the running max moves
constexpr int kAccPad = 132;      // LDS row pitch (floats) for the wave merge
constexpr int kNoTokens = 1 << 30;  // token base of a position with nothing to read

// One wave's 32-token chunk of a (page, KV head) block as loaded: 1 KiB
// rows of K and V, 16 bytes per lane each (FP8: 4 rows of each, every
// 16-byte piece two 8-byte operands; bf16: 8 rows, every piece one
// operand), plus the chunk's per-token scales.
template <bool BF>
struct Chunk {
  static constexpr int kRows = BF ? 8 : 4;
  u32x4 k[kRows];
  u32x4 v[kRows];
  f32x4 ks[2];
  f32x4 vs[2];
};

// Request of a query row: largest b with cu[b] <= row.
__device__ __forceinline__ int find_request(const int32_t* cu, int batch, int row) {
  int lo = 0, hi = batch;  // answer in [0, batch)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// Rows [start, start + L) of request b from cu_seqlens_q, clamped into
// [0, rows) so that a malformed cu can only give wrong values, never an
// access outside q or out.
__device__ __forceinline__ void request_rows(const DecodeArgs& a, int b, int* start, int* L) {
  const int s = min(max(a.cu_seqlens_q[b], 0), a.rows);
  const int e = min(max(a.cu_seqlens_q[b + 1], s), a.rows);
  *start = s;
  *L = e - s;
}

// Length-balanced partitions (dense calls of at most 64 requests; lane j
// stands for request j).  Every partition of the call holds ppp pages:
// the smallest ppp for which the requests' partitions, max(1, ceil(pages_j
// / ppp)) each, fit the nslot launched slots.  ppp is found by bisection
// between ceil(total / nslot) and ceil(total / (nslot - batch)); the upper
// end always fits, since the partitions then number at most total / ppp +
// batch.  Slots go to the requests in order.  The main and the merge kernel
// both derive this from the context lengths, so they agree without a pass
// of their own.
struct Balanced {
  int ppp;    // pages per partition
  int first;  // lane j: first slot of request j
  int parts;  // lane j: partitions of request j (0 past the batch)
  int ctx;    // lane j: context length of request j
};

__device__ __forceinline__ Balanced balanced_layout(const DecodeArgs& a) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool live = lane < a.batch;
  Balanced r;
  r.ctx = live ? a.context_lens[lane] : 0;
  const int np = (max(0, min(r.ctx, a.width * 128)) + 127) >> 7;  // pages the request's last row sees
  const int total = int(wave_reduce_u32<UOp::ADD>(uint32_t(np)));
  // max(1, ceil(np / ppp)) per request.  np <= 2^20, so the float quotient
  // (exact operands below 2^24, a reciprocal within 2 ulp) is within one of
  // floor((np + ppp - 1) / ppp), and one correction each way makes it exact;
  // this is a third of the instructions of a 32-bit integer division.
  auto parts_at = [&](int ppp) {
    const uint32_t n = uint32_t(np + ppp - 1), d = uint32_t(ppp);
    uint32_t q = uint32_t(float(n) * __builtin_amdgcn_rcpf(float(d)));
    const int32_t r = int32_t(n - q * d);
    q = r < 0 ? q - 1 : (uint32_t(r) >= d ? q + 1 : q);
    return live ? max(1, int(q)) : 0;
  };
  int lo = max(1, (total + a.nslot - 1) / a.nslot);
  int hi = max(lo, (total + a.nslot - a.batch - 1) / (a.nslot - a.batch));
  // equal lengths that divide evenly fit at the lower end: one count, no search
  if (hi > lo && int(wave_reduce_u32<UOp::ADD>(uint32_t(parts_at(lo)))) <= a.nslot) hi = lo;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (int(wave_reduce_u32<UOp::ADD>(uint32_t(parts_at(mid)))) <= a.nslot) hi = mid;
    else lo = mid + 1;
  }
  r.ppp = lo;
  r.parts = parts_at(lo);
  r.first = wave_inclusive_scan(r.parts) - r.parts;
  return r;
}

__device__ __forceinline__ int lane_int(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// An empty asm that reads every register of a chunk: forces the compiler to
// complete the chunk's loads here (used on paths that skip the chunk).
template <bool PER_TOKEN, bool BF>
__device__ __forceinline__ void consume_chunk(const Chunk<BF>& c) {
#pragma unroll
  for (int i = 0; i < Chunk<BF>::kRows; ++i) asm volatile("" ::"v"(c.k[i]), "v"(c.v[i]));
  if constexpr (PER_TOKEN) asm volatile("" ::"v"(c.ks[0]), "v"(c.ks[1]), "v"(c.vs[0]), "v"(c.vs[1]));
}

// Per-wave byte offsets of a lane's loads inside a block: the 16-byte
// piece of its chunk, and the first of its 8 tokens' scales.
struct LaneOffsets {
  int kv;     // chunk * chunk_bytes + 16 * lane
  int scale;  // 4 * (32 * chunk + 4 * (lane / 16))
};
template <bool BF>
__device__ __forceinline__ LaneOffsets lane_offsets(int chunk, int lane) {
  constexpr int kChunkBytes = BF ? 8192 : 4096;  // one 32-token chunk of a block
  return LaneOffsets{chunk * kChunkBytes + 16 * lane, 4 * (32 * chunk + 4 * (lane >> 4))};
}

// Loads one wave's 32-token chunk of (page, KV head) block `blk` through
// buffer resources whose base is the block: the block address stays in
// scalar registers, every lane's offset is fixed per wave, and the four
// (FP8) or eight (bf16) 1 KiB rows are immediate offsets -- no per-load
// address arithmetic.  When `valid` is false the resources cover 0 bytes:
// the same loads are issued (so the compiler's wait counts stay exact across
// the prefetch ring) but they return zeros and touch no memory.
template <bool PER_TOKEN, bool BF, bool ONCE>
__device__ __forceinline__ void load_chunk(Chunk<BF>& c, const DecodeArgs& a, int64_t blk, bool valid,
                                           LaneOffsets lo) {
  constexpr int kBlockBytes = BF ? 32768 : 16384;  // one (page, head) block
  const int64_t b = valid ? blk : 0;
  const int nrec = valid ? kBlockBytes : 0;
  const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.k_cache + b * kBlockBytes, nrec);
  const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.v_cache + b * kBlockBytes, nrec);
  // ONCE: these K and V bytes are read once per call (one-row workgroups)
  // or by at most two row groups, so non-temporal loads keep them from
  // evicting what is reused (tables, the split-K partials the merge reads
  // next, the pages the writer touches).  With more row groups per page the
  // later groups' reads should hit the cache.
  constexpr int kAux = ONCE ? 2 : 0;  // cache-policy bit 1: non-temporal
#pragma unroll
  for (int i = 0; i < Chunk<BF>::kRows; ++i)
    c.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, lo.kv + 1024 * i, 0, kAux);
#pragma unroll
  for (int i = 0; i < Chunk<BF>::kRows; ++i)
    c.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, lo.kv + 1024 * i, 0, kAux);
  if constexpr (PER_TOKEN) {
    const int sn = valid ? 512 : 0;  // 128 fp32 scales per block
    const __amdgpu_buffer_rsrc_t rks = block_rsrc(a.k_scale + b * 128, sn);
    const __amdgpu_buffer_rsrc_t rvs = block_rsrc(a.v_scale + b * 128, sn);
    c.ks[0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, lo.scale, 0, 0));
    c.ks[1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, lo.scale + 64, 0, 0));
    c.vs[0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, lo.scale, 0, 0));
    c.vs[1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, lo.scale + 64, 0, 0));
  }
}


// Two workgroups per CU (256 registers per lane) for the four-wave,
// two-page-ring shapes; one for the rest -- including two-row bf16, whose
// two 16 KiB-per-wave chunk buffers and two rows of accumulators need more.
template <int RT, bool NBUF2_NW4, bool BF>
constexpr int kMinBlocks = (NBUF2_NW4 && !(BF && RT == 2)) ? 2 : 1;

// In-kernel log-sum-exp merge.  Every partition of a unit (request or
// row, KV head, row group) bumps the unit's counter once its partial is
// visible to the whole device; the partition that sees parts-1 knows every
// partial is written and merges them (the same arithmetic as pa_merge, in
// partition order), then puts the counter back to 0 for the next call.
// Threads < 256: (head oh, 8 dims od) as in the wave merge.  sm_w holds
// 16 x kMaxParts weights (LDS of the finished wave merge).
constexpr int kMaxMergeParts = 256;

// Partials of the in-kernel merge travel through device-scope (relaxed
// atomic) 64-bit stores and loads, which are coherent across the XCDs' L2s;
// the arrival count orders them (acquire-release, see merge_if_last).
__device__ __forceinline__ void store_coherent(float* p, float x, float y) {
  const uint64_t v = uint64_t(__float_as_uint(x)) | (uint64_t(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float(uint32_t(v)), __uint_as_float(uint32_t(v >> 32))};
}
// s_waitcnt vmcnt(0): every vector memory operation of this wave -- here
// the coherent partial stores -- has completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }
constexpr int kMergeChunk = 8;  // partitions whose accumulators are loaded together

__device__ void merge_if_last(const DecodeArgs& a, int64_t unit, int row0, int nrows, int h, float* sm_w) {
  __shared__ int sm_last;
  // Each wave waits for its coherent partial stores to complete, the
  // barrier makes that true for the whole workgroup, and only then does
  // thread 0 count the partition in.  The count is an acquire-release
  // read-modify-write at device scope: it publishes this workgroup's
  // partials (release) and, for the workgroup that sees the last arrival,
  // orders every other partition's published partials before its reads
  // (acquire); the barrier after it carries that order to the other waves.
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(a.unit_count + unit, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
              uint32_t(a.parts - 1);
  __syncthreads();
  if (!sm_last) return;
  const int t = threadIdx.x;
  const int li = t & 15;          // this thread's share of the partitions: li, li+16, ...
  const int oh = (t >> 4) & 15;
  const int od = li * 8;
  const int P = a.parts;
  const int Hq = 16 * a.hkv;
  const int64_t stride_p = int64_t(a.rows) * Hq;
  float v_fold = 1.0f;
  if (a.scale_mode != PA_SCALE_PER_TOKEN && a.v_scale) v_fold = *a.v_scale;
  for (int r = 0; r < nrows; ++r) {
    const int row = row0 + r;
    const int64_t base = int64_t(row) * Hq + 16 * h + oh;
    float M = -INFINITY, L = 0.0f;
    if (t < 256) {
      float2 ml[kMaxMergeParts / 16];
#pragma unroll
      for (int i = 0; i < kMaxMergeParts / 16; ++i) {
        const int p = li + 16 * i;
        ml[i] = p < P ? load_coherent(a.part_ml + 2 * (p * stride_p + base)) : float2{-INFINITY, 0.0f};
        M = fmaxf(M, ml[i].x);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 16));
#pragma unroll
      for (int i = 0; i < kMaxMergeParts / 16; ++i) {
        const int p = li + 16 * i;
        const float w = (M == -INFINITY || ml[i].x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml[i].x - M);
        L += w * ml[i].y;
        if (p < P) sm_w[oh * kMaxMergeParts + p] = w;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) L += __shfl_xor(L, o, 16);
    }
    __syncthreads();
    if (t < 256) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      for (int p0 = 0; p0 < P; p0 += kMergeChunk) {
        f32x4 v0[kMergeChunk], v1[kMergeChunk];
#pragma unroll
        for (int j = 0; j < kMergeChunk; ++j) {
          const int p = min(p0 + j, P - 1);
          const float* ap = a.part_acc + (p * stride_p + base) * 128 + od;
          const float2 x0 = load_coherent(ap), x1 = load_coherent(ap + 2);
          const float2 x2 = load_coherent(ap + 4), x3 = load_coherent(ap + 6);
          v0[j] = f32x4{x0.x, x0.y, x1.x, x1.y};
          v1[j] = f32x4{x2.x, x2.y, x3.x, x3.y};
        }
#pragma unroll
        for (int j = 0; j < kMergeChunk; ++j) {
          // an empty partition has weight 0 and unwritten accumulators: skip, never multiply
          const float w = p0 + j < P ? sm_w[oh * kMaxMergeParts + p0 + j] : 0.0f;
          if (w != 0.0f) {
            s0 += w * v0[j];
            s1 += w * v1[j];
          }
        }
      }
      const float inv = L > 0.0f ? v_fold / L : 0.0f;
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        packed[e] = uint32_t(f32_to_bf16_rne(s0[2 * e] * inv)) | (uint32_t(f32_to_bf16_rne(s0[2 * e + 1] * inv)) << 16);
        packed[2 + e] =
            uint32_t(f32_to_bf16_rne(s1[2 * e] * inv)) | (uint32_t(f32_to_bf16_rne(s1[2 * e + 1] * inv)) << 16);
      }
      uint16_t* op = a.out + int64_t(row) * a.out_row_stride + int64_t(16 * h + oh) * a.out_head_stride + od;
      *reinterpret_cast<u32x4*>(op) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
    __syncthreads();
  }
  if (t == 0) __hip_atomic_store(a.unit_count + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup id -> (unit q, row group gi) of a dense grid with several row
// groups per unit.  With at least 8 units, id x + 8s carries row group
// s % groups of unit 8(s / groups) + x: ids go round-robin over the 8 XCDs,
// so the groups of one unit are consecutive dispatches on one XCD and the
// second read of each page is an L2 hit.  With fewer than 8 units (long
// q_len over few requests, e.g. a prompt run as one request) that layout
// would leave XCDs idle, so the ids run over (row group, unit) with the unit
// fastest and every XCD gets row groups.
__device__ __forceinline__ void xcd_group_of(const DecodeArgs& a, uint32_t* q, int* gi) {
  if (a.nq < 8) {
    *q = blockIdx.x % uint32_t(a.nq);
    *gi = int(blockIdx.x / uint32_t(a.nq));
  } else {
    const uint32_t x = blockIdx.x & 7u, s = blockIdx.x >> 3;
    *gi = int(s % uint32_t(a.groups));
    *q = (s / uint32_t(a.groups)) * 8u + x;
  }
}

// ONCE2: a two-row workgroup's K/V loads are non-temporal (a.kv_once).
template <int RT, bool PER_TOKEN, bool SPARSE, int NBUF, int NW, bool BF, bool FW, bool ONCE2>
__global__ __launch_bounds__(kWave * NW, (kMinBlocks<RT, NW == 4 && NBUF <= 2, BF>)) void pa_decode_main(
    DecodeArgs a) {
  static_assert(!(BF && PER_TOKEN), "a bf16 cache carries no scales");
  static_assert(!(FW && SPARSE) || (RT == 1 && NW == 4), "the sparse fused write: one row, four waves");
  static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
  static_assert(!ONCE2 || RT == 2, "one-row workgroups always load non-temporally");
  constexpr bool kOnce = RT == 1 || ONCE2;
  static_assert(NW * 16 * kAccPad >= 16 * kMaxMergeParts, "merge weights reuse the wave-merge LDS");
  static_assert((kWave * NW) % 256 == 0, "the combine takes 256 threads per row");
  __shared__ float sm_ml[NW][RT][16][2];
  __shared__ float sm_acc[RT][NW][16][kAccPad];  // per row, per wave
  constexpr int S = NW / 4;  // pages streamed side by side (one per group of four waves)
  const int lane = threadIdx.x & (kWave - 1);
  // wave index as a provably uniform (scalar) value: table reads indexed by
  // it stay scalar loads, off the vector-memory counter of the KV stream
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int cw = wave & 3;   // 32-token chunk of each page this wave handles
  const int ps = wave >> 2;  // page stream: positions n0 + ps, n0 + ps + S, ...
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of each 16-token tile
  const int hr = lane & 15;  // query head within the GQA group
  const LaneOffsets lofs = lane_offsets<BF>(cw, lane);
  const int Hq = 16 * a.hkv;

  int part;
  int64_t unit = 0;
  int ppp = a.ppp;
  int bal_slot = 0, bal_b = 0, bal_h = 0, bal_gi = 0, bal_ctx = 0;
  if (!SPARSE && a.balanced) {
    // slot (a partition position shared by the requests), KV head, row group
    uint32_t slot;
    if (a.xcd_grouped) {
      // as below: the row groups of one (slot, KV head) on one XCD
      uint32_t q;
      xcd_group_of(a, &q, &bal_gi);
      if (q >= uint32_t(a.nq)) return;
      slot = q / uint32_t(a.hkv);
      bal_h = int(q % uint32_t(a.hkv));
    } else {
      slot = blockIdx.x / uint32_t(a.hkv);
      bal_h = int(blockIdx.x % uint32_t(a.hkv));
    }
    const Balanced bl = balanced_layout(a);
    // the request whose slots hold this one: the requests before it are
    // those whose slots end at or before it
    bal_b = __builtin_popcountll(
        __builtin_amdgcn_ballot_w64(lane < a.batch && bl.first + bl.parts <= int(slot)));
    if (bal_b >= a.batch) return;  // past the last request's partitions
    bal_slot = int(slot);
    part = int(slot) - lane_int(bl.first, bal_b);
    bal_ctx = lane_int(bl.ctx, bal_b);
    ppp = bl.ppp;
  } else if (!SPARSE && a.xcd_grouped) {
    // Row groups of one (request, KV head, partition) read the same pages:
    // give them workgroup ids x + 8s, x + 8(s+1), ... -- consecutive
    // dispatches on the same XCD (ids go round-robin over the 8 XCDs), so
    // the second read of each page is an L2 hit.
    uint32_t q;  // (partition, request, KV head)
    int gi;
    xcd_group_of(a, &q, &gi);
    if (q >= uint32_t(a.nq)) return;  // padding of the last XCD round
    const uint32_t nbh = uint32_t(a.nq / a.parts);
    part = int(q / nbh);
    unit = int64_t(q % nbh) * a.groups + gi;
  } else {
    // partition-major: every request's first partitions (full ones) are
    // dispatched before later (partial or empty) ones, so when there are
    // more workgroups than slots the dispatcher hands the short ones to the
    // CUs that finish first
    const uint32_t units = uint32_t(gridDim.x / uint32_t(a.parts));
    part = int(blockIdx.x / units);
    unit = blockIdx.x % units;
  }

  // ---- which rows, which request, which tokens -------------------------
  // The loads that decide the partition's work (context length, row range,
  // the partition's first block-table entry) are issued together, before
  // any branch, so they cost one memory round trip.
  const int n0 = part * ppp;  // < width (dense) or < topk (sparse) by construction of the grid
  const int s0 = n0 + ps;       // this wave's first list position
  int h, b, row0, nrows, lim0;  // row row0+i sees tokens t < lim0 + i (fused write: t < lim0)
  int fz_start = 0, fz_L = 0, fz_ctx = 0, fz_i0 = 0;  // request rows, length, context; group's first row
  int first_entry;              // dense: block_table[b][s0]; sparse: sparse_idx[row0][s0] (-1 past the end)
  int second_entry = -1;        // dense: block_table[b][s0 + S], read with the first
  if constexpr (SPARSE) {
    h = int(unit % a.hkv);
    row0 = int(unit / a.hkv);
    first_entry = s0 < a.topk ? as_const(a.sparse_idx + int64_t(row0) * a.sp_stride)[s0] : -1;
    int start, L;
    if (a.cu_seqlens_q) {
      b = find_request(a.cu_seqlens_q, a.batch, row0);
      request_rows(a, b, &start, &L);
    } else {
      L = a.uniform_q_len;
      b = row0 / L;
      start = b * L;
    }
    nrows = 1;
    const int ctx = a.context_lens[b];
    // the sparse fused write serves single-row requests: the row's own new
    // token (position ctx - 1) is attended separately, when its page is on
    // the row's list
    lim0 = FW ? ctx - L + (row0 - start) : ctx - L + (row0 - start) + 1;
    if constexpr (FW) {
      fz_start = row0;
      fz_L = 1;
      fz_ctx = ctx;
      fz_i0 = 0;
    }
  } else {
    int gi;
    if (a.balanced) {
      gi = bal_gi;
      h = bal_h;
      b = bal_b;
    } else {
      gi = int(unit % a.groups);
      const int64_t bh = unit / a.groups;
      h = int(bh % a.hkv);
      b = int(bh / a.hkv);
    }
    first_entry = s0 < a.width ? as_const(a.block_table + int64_t(b) * a.bt_stride)[s0] : -1;
    // the next position's entry travels with the first: its page's loads
    // need not wait for a second table round trip after the context length
    second_entry = s0 + S < a.width ? as_const(a.block_table + int64_t(b) * a.bt_stride)[s0 + S] : -1;
    const int ctx = a.balanced ? bal_ctx : a.context_lens[b];
    int start, L;
    if (a.cu_seqlens_q) {
      request_rows(a, b, &start, &L);
    } else {
      L = a.uniform_q_len;
      start = b * L;
    }
    const int i0 = gi * RT;
    if (i0 >= L) return;  // this request has no rows in this group
    nrows = min(RT, L - i0);
    row0 = start + i0;
    // with the fused write every row of the main loop sees only the older
    // positions; the request's new tokens are attended separately
    lim0 = FW ? ctx - L : ctx - L + i0 + 1;
    fz_start = start;
    fz_L = L;
    fz_ctx = ctx;
    fz_i0 = i0;
  }
  // Fused write: the partition holding the request's last attended position
  // takes the new tokens.  Each wave's first new token is loaded ahead of
  // the page stream, quantized and stored while the first pages load, and
  // attended after the stream.  The loads are issued by every wave (a wave
  // past the request's tokens reloads its last one), so the compiler counts
  // them exactly and waits for them alone.
  bool fz_last = false;
  float fk0 = 0.f, fk1 = 0.f, fv0 = 0.f, fv1 = 0.f;
  int64_t fslot = -1;
  // Sparse: which partition holds the new token's page is known only from
  // the list, so wave 0 of every workgroup takes the token; partition 0
  // stores it, and the workgroup whose stream passes its page attends it.
  const int fz_page_base = (fz_ctx - 1) >> 7 << 7;  // token base of the new token's page (sparse)
  bool fz_seen = false;
  float fz_ksc = 1.0f, fz_vsc = 1.0f;  // SCALAR mode: the caller's scales (scalar loads)
  if constexpr (FW) {
    const int ctx_cap = min(fz_ctx, a.width * 128);
    const int pl = (ctx_cap - 1) >> 7;
    fz_last = ctx_cap > 0 && n0 <= pl && pl < n0 + ppp;
    const int64_t t = fz_start + min(wave, max(fz_L, 1) - 1);
    load_pair(a.k_new, t * a.kn_tok_stride + h * a.kn_head_stride + 2 * lane, a.kn_bf16, &fk0, &fk1);
    load_pair(a.v_new, t * a.vn_tok_stride + h * a.vn_head_stride + 2 * lane, a.kn_bf16, &fv0, &fv1);
    fslot = a.slots[t];
    if (!BF && a.scale_mode == PA_SCALE_SCALAR) {
      fz_ksc = __int_as_float(as_const(reinterpret_cast<const int32_t*>(a.k_scale))[0]);
      fz_vsc = __int_as_float(as_const(reinterpret_cast<const int32_t*>(a.v_scale))[0]);
    }
  }
  const bool fz_pend = fz_last && wave < fz_L;  // this wave has a first new token
  // the wave that quantizes and stores its first token before the stream
  const bool fz_mine = SPARSE ? wave == 0 : fz_pend;

  // The partition's first chunk and the query operands do not depend on the
  // context length: issue their loads now, so they travel together with the
  // context-length read instead of after it (masking handles the rest).
  Chunk<BF> buf[NBUF];
  int tb[NBUF];
  {
    int ln0 = s0, P0 = first_entry;
    if constexpr (SPARSE) {
      ln0 = first_entry;
      P0 = (ln0 >= 0 && ln0 < a.width) ? as_const(a.block_table + int64_t(b) * a.bt_stride)[ln0] : -1;
    }
    const bool ok0 = P0 >= 0 && P0 < a.num_blocks;
    tb[0] = ok0 ? ln0 * 128 : kNoTokens;
    load_chunk<PER_TOKEN, BF, kOnce>(buf[0], a, int64_t(P0) * a.hkv + h, ok0, lofs);
  }
  // query operands: B of S^T = K Q^T, lane = (head hr, dims 8g..8g+7 of
  // each 32-dim k-step)
  // A workgroup with fewer rows than RT (the last group of an odd q_len)
  // computes its missing row as a copy of its last real row and never writes
  // it: the per-chunk code then has no per-row branches, so the scheduler
  // can interleave the rows' MFMA chains.
  static_assert(RT == 1 || RT == 2, "a workgroup carries one or two query rows");
  bf16x8 qop[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* qp = a.q + int64_t(row0 + min(r, nrows - 1)) * a.q_row_stride +
                           int64_t(16 * h + hr) * a.q_head_stride + 32 * j + 8 * g;
      qop[r][j] = *reinterpret_cast<const bf16x8*>(qp);
    }
  }

  const int cap = a.width * 128;
  const int rstep = FW ? 0 : 1;  // cutoff step from one row to the next
  const int lim_min = max(0, min(lim0, cap));
  const int lim_max = max(0, min(lim0 + (nrows - 1) * rstep, cap));

  int n1;
  if constexpr (SPARSE) {
    n1 = min(n0 + ppp, a.topk);
  } else {
    const int npages = (lim_max + 127) >> 7;
    n1 = min(n0 + ppp, npages);
  }
  // where this workgroup's rows leave their partials: partition-major over
  // all rows, or (balanced) slot-major over the rows of one request
  const bool to_partial = a.balanced || a.parts > 1;
  const int64_t prow0 = a.balanced ? int64_t(bal_slot) * a.lrows + bal_gi * RT : int64_t(part) * a.rows + row0;
  if (n0 >= n1 && to_partial && !fz_last) {
    // nothing to attend in this partition: leave an empty partial (weight 0)
    // so the merge can read every partition without knowing the context
    if (threadIdx.x < 16 * nrows) {
      const int r = threadIdx.x >> 4;
      const int64_t pi = (prow0 + r) * Hq + 16 * h + (threadIdx.x & 15);
      if (a.unit_count) store_coherent(a.part_ml + 2 * pi, -INFINITY, 0.0f);
      else *reinterpret_cast<float2*>(a.part_ml + 2 * pi) = float2{-INFINITY, 0.0f};
    }
    if (a.unit_count) merge_if_last(a, unit, row0, nrows, h, &sm_acc[0][0][0][0]);
    return;
  }

  float k_fold = a.sm_log2;  // scalar / none: the K scale folds into the score scale
  float v_fold = 1.0f;       // ... and the V scale into the normalized output
  if constexpr (!PER_TOKEN) {
    if (a.k_scale) k_fold *= *a.k_scale;
    if (a.v_scale) v_fold = *a.v_scale;
  }

  f32x4 acc[RT][8];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[r][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const_i32_ptr bt_c = as_const(a.block_table + int64_t(b) * a.bt_stride);
  const_i32_ptr sp_c = nullptr;
  if constexpr (SPARSE) sp_c = as_const(a.sparse_idx + int64_t(row0) * a.sp_stride);
  // Table reads are split in two so that a scalar load is never waited for
  // in the step that issues it: raw_at() issues the read of list position n
  // (its physical page), valid_page() checks it one step later.
  // logical page of list position n (sparse: the list entry; -1 past the end)
  auto logical_at = [&](int n) -> int {
    if constexpr (SPARSE) return n < n1 ? (n == s0 ? first_entry : sp_c[n]) : -1;
    return n;
  };
  // (sparse fused write: the page that starts with the row's new token is
  // still streamed -- its bytes are all masked -- so that the stream sees
  // it is on the list)
  constexpr int kListSlack = (FW && SPARSE) ? 1 : 0;
  auto logical_ok = [&](int n, int ln) -> bool {
    return n < n1 && ln >= 0 && ln < a.width && ln * 128 < lim_max + kListSlack;
  };
  // raw physical page of logical page ln (read only if the position is usable)
  auto raw_at = [&](int n, int ln) -> int {
    if (!logical_ok(n, ln)) return -1;
    if constexpr (!SPARSE) {
      if (n == s0) return first_entry;
      if (n == s0 + S) return second_entry;
    }
    return bt_c[ln];
  };
  auto valid_page = [&](int P) -> bool { return P >= 0 && P < a.num_blocks; };
  auto process = [&](Chunk<BF>& c, int tbase) {
    if constexpr (FW && SPARSE) fz_seen = fz_seen || tbase == fz_page_base;
    const int t0 = tbase + 32 * cw;
    if (t0 >= lim_max) {
      // nothing of this chunk is attended: still consume its registers so the
      // loads are complete on this path too
      consume_chunk<PER_TOKEN, BF>(c);
      return;
    }
    const bool full = t0 + 32 <= lim_min;

    // token of this lane's score slot e: t0 + 16*(e/4) + 4g + e%4
    if (!full) {
      keep_branch();
      // One row: V scales of tokens past its cutoff become 0 (in the loaded
      // registers); their scores are -inf, so p = 0, and p * 0 stays 0
      // whatever an unwritten slot holds.  (Two rows mask P' per row below:
      // the first row stops one token before the second, whose newest token
      // has a written scale that need not be finite.  Without per-token
      // scales p = 0 alone gives P' = 0.)
      if constexpr (PER_TOKEN && RT == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) >= lim_max) c.vs[e >> 2][e & 3] = 0.0f;
      }
      // zero V of tokens past the context: those slots were never written
      // (a NaN there would survive a zero weight in the product)
      if constexpr (BF) {
        // word w holds slots 2w, 2w+1 of one dim
        uint32_t m[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          m[w] = 0;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int e = 2 * w + s2;
            if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) < lim_max) m[w] |= 0xFFFFu << (16 * s2);
          }
        }
#pragma unroll
        for (int i = 0; i < Chunk<BF>::kRows; ++i) {
          c.v[i][0] &= m[0]; c.v[i][1] &= m[1]; c.v[i][2] &= m[2]; c.v[i][3] &= m[3];
        }
      } else {
        // bytes 0-3 of a dword: slots 0-3 (first 16 tokens), next dword slots 4-7
        uint32_t m0 = 0, m1 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (t0 + 4 * g + e < lim_max) m0 |= 0xFFu << (8 * e);
          if (t0 + 16 + 4 * g + e < lim_max) m1 |= 0xFFu << (8 * e);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c.v[i][0] &= m0; c.v[i][1] &= m1; c.v[i][2] &= m0; c.v[i][3] &= m1;
        }
      }
    }

    // per-token factors of this lane's 8 tokens (slot e <-> token
    // t0 + 16*(e/4) + 4g + e%4): K scale folded with sm*log2(e), V scale
    float kc[8], vsf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (PER_TOKEN) {
        kc[e] = c.ks[e >> 2][e & 3] * k_fold;
        vsf[e] = c.vs[e >> 2][e & 3];
      } else {
        kc[e] = k_fold;
        vsf[e] = 1.0f;
      }
    }

    // Two-row workgroups run two waves per SIMD.  A wave raises its issue
    // priority while it issues its MFMA blocks, so the SIMD hands them to it
    // ahead of the other wave's softmax instructions and the matrix pipe
    // runs under that wave's VALU work instead of after it.  The QK block,
    // which starts a chunk's dependency chain, goes first (2), then P.V (1).
    if constexpr (RT == 2) __builtin_amdgcn_s_setprio(2);
    // S^T = K Q^T for every row tile, k-step outer so each converted K
    // operand (exact e4m3 -> bf16, or the bf16 itself) serves all row tiles
    f32x4 st[RT][2];
#pragma unroll
    for (int r = 0; r < RT; ++r) st[r][0] = st[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 k0, k1;  // k-step j of the first and second 16-token tile
      if constexpr (BF) {
        k0 = __builtin_bit_cast(bf16x8, c.k[j]);
        k1 = __builtin_bit_cast(bf16x8, c.k[4 + j]);
      } else {
        k0 = fp8x8_to_bf16x8(c.k[j >> 1][2 * (j & 1)], c.k[j >> 1][2 * (j & 1) + 1]);
        k1 = fp8x8_to_bf16x8(c.k[2 + (j >> 1)][2 * (j & 1)], c.k[2 + (j >> 1)][2 * (j & 1) + 1]);
      }
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const bf16x8 qv = qop[r][j];
        st[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qv, st[r][0], 0, 0, 0);
        st[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qv, st[r][1], 0, 0, 0);
      }
    }

    if constexpr (RT == 2) __builtin_amdgcn_s_setprio(0);

    // online softmax per row tile; P' = p * v_scale as a bf16 hi + lo pair:
    // hi keeps the top 8 significant bits (truncation), lo = P' - hi is exact
    // in fp32 and rounds to bf16, so the pair carries ~16 bits -- the PV
    // product then adds no rounding beyond fp32 accumulation order.
    bf16x8 phi[RT], plo[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      // scores relative to the running max (0 before the row has one): the
      // subtraction rides in the fma, and the lazy test is on x directly
      const float mu = (m_run[r] == -INFINITY) ? 0.0f : m_run[r];
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = fmaf(st[r][0][e], kc[e], -mu);
        x[4 + e] = fmaf(st[r][1][e], kc[4 + e], -mu);
      }
      const int lim_r = min(lim0 + min(r, nrows - 1) * rstep, cap);
      if (!full) {
        keep_branch();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = t0 + 16 * (e >> 2) + 4 * g + (e & 3);
          x[e] = t < lim_r ? x[e] : -INFINITY;
        }
      }
      const float lm = max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), max2f(x[6], x[7]));
      const bool need = lm > (m_run[r] == -INFINITY ? -INFINITY : kLazyMax);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        float gm = fmaxf(lm, __shfl_xor(lm, 16, kWave));
        gm = fmaxf(gm, __shfl_xor(gm, 32, kWave));
        const float mn = fmaxf(m_run[r], gm + mu);
        const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - mn);
        l_run[r] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[r][d] *= alpha;
        m_run[r] = mn;
        // re-base the chunk's scores on the new max
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
      if (PER_TOKEN && RT == 2 && !full) {
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
      // pairwise sum: three dependent adds instead of eight
      l_run[r] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
      u32x4 hw;
#pragma unroll
      for (int e = 0; e < 4; ++e) hw[e] = __builtin_amdgcn_perm(hb[2 * e + 1], hb[2 * e], 0x07060302u);
      phi[r] = __builtin_bit_cast(bf16x8, hw);
#pragma unroll
      for (int e = 0; e < 8; ++e) plo[r][e] = (__bf16)lo[e];
    }

    if constexpr (RT == 2) __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P'^T, d-tile outer so each converted V operand serves all
    // row tiles
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      bf16x8 vop;  // dims 16d..16d+15 of the chunk's 32 tokens
      if constexpr (BF) vop = __builtin_bit_cast(bf16x8, c.v[d]);
      else vop = fp8x8_to_bf16x8(c.v[d >> 1][2 * (d & 1)], c.v[d >> 1][2 * (d & 1) + 1]);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        acc[r][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi[r], acc[r][d], 0, 0, 0);
        acc[r][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo[r], acc[r][d], 0, 0, 0);
      }
    }
    if constexpr (RT == 2) __builtin_amdgcn_s_setprio(0);
  };

  // ---- the request's new tokens (fused write) -------------------------------
  // Wave w takes new tokens w, w + NW, ...: it quantizes the token's K and V
  // rows exactly as kv_quant_write does (writer_common.h), stores them when
  // this is row group 0 (one store per token), and folds the token into its
  // own (max, sum, accumulators) for the rows that see it -- row i of the
  // request sees new tokens 0..i.  The dequantized codes go through this
  // wave's LDS rows (untouched until the epilogue) from the writer's layout
  // (two dims per lane) to the score layout (the query operand's dims) and
  // the accumulator layout, a few values at a time.  Scores and weights are
  // fp32: the token's K scale multiplies its score, its V scale its weight,
  // as in the page stream.  A wave's first token is quantized and stored
  // before the page stream (under the first pages' loads) and folded in
  // after it; folding it inside the stream's first step measured slower
  // (more registers live through the loop).
  // Quantize (bf16 cache: round) this lane's two K and two V values of a
  // new token and store them if asked; returns the stored values: FP8 codes
  // (low 16 bits) or bf16 pairs, and the scales through ks_t, vs_t.
  auto write_token = [&](float k0, float k1, float v0, float v1, int64_t slot, bool store, uint32_t* kw,
                         uint32_t* vw, float* ks_t, float* vs_t) __attribute__((always_inline)) {
    if constexpr (FW) {
      if constexpr (BF) {
        // the unquantized cache: the elements rounded to bf16, no scale
        *kw = f32_to_bf16_bits(k0) | (f32_to_bf16_bits(k1) << 16);
        *vw = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
        *ks_t = *vs_t = 1.0f;
        if (store && slot >= 0 && slot < a.num_blocks * 128)
          store_token_bf16(a.k_cache_w, a.v_cache_w, a.hkv, slot, h, lane, *kw, *vw);
      } else {
        *kw = quantize_pair_v(k0, k1, a.scale_mode, fz_ksc, ks_t);
        *vw = quantize_pair_v(v0, v1, a.scale_mode, fz_vsc, vs_t);
        if (store && slot >= 0 && slot < a.num_blocks * 128)
          store_token_fp8(a.k_cache_w, a.v_cache_w, a.k_scale_w, a.v_scale_w, a.hkv, a.scale_mode, slot, h, lane,
                          *kw, *vw, *ks_t, *vs_t);
      }
    }
  };
  // Fold new token j (values as write_token returned them) into the rows
  // that see it.
  auto fold_token = [&](int j, uint32_t kw, uint32_t vw, float ks_t, float vs_t) __attribute__((always_inline)) {
    if constexpr (FW) {
      float* lds = &sm_acc[0][wave][0][0];  // 256 floats: the K codes' values, then V's
      bf16x2 kb, vb;  // the stored values: the dequantized codes, or the bf16 elements
      if constexpr (BF) {
        kb = __builtin_bit_cast(bf16x2, kw);
        vb = __builtin_bit_cast(bf16x2, vw);
      } else {
        kb = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw, 1.0f, false);
        vb = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw, 1.0f, false);
      }
      const int pos = fz_ctx - fz_L + j;
      if (pos < 0 || pos >= cap) return;  // not attended (uniform)
      // the previous token's reads of these rows are done before they change
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      *reinterpret_cast<float2*>(lds + 2 * lane) = float2{float(kb[0]), float(kb[1])};
      *reinterpret_cast<float2*>(lds + 128 + 2 * lane) = float2{float(vb[0]), float(vb[1])};
      // the wave's LDS writes complete before any lane reads another's
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float kcf = PER_TOKEN ? ks_t * k_fold : k_fold;
      const float vsf = PER_TOKEN ? vs_t : 1.0f;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        if (r >= nrows || j > fz_i0 + r) continue;  // uniform: this row does not see token j
        float s = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 lo4 = *reinterpret_cast<const f32x4*>(lds + 32 * jj + 8 * g);
          const f32x4 hi4 = *reinterpret_cast<const f32x4*>(lds + 32 * jj + 8 * g + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s = fmaf(float(qop[r][jj][i]), lo4[i], s);
            s = fmaf(float(qop[r][jj][4 + i]), hi4[i], s);
          }
        }
        s += __shfl_xor(s, 16, kWave);  // the head's four lane groups hold its 128 dims
        s += __shfl_xor(s, 32, kWave);
        const float sc = s * kcf;  // log2-domain score, equal in the head's four lanes
        // raise the running max as the page stream does: lazily, so p <= 2^8
        const bool raise = m_run[r] == -INFINITY || sc - m_run[r] > kLazyMax;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float mn = raise ? fmaxf(m_run[r], sc) : m_run[r];
          const float alpha = (m_run[r] == -INFINITY || !raise) ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - mn);
          l_run[r] *= alpha;
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[r][d] *= alpha;
          m_run[r] = mn;
        }
        const float p = __builtin_amdgcn_exp2f(sc - m_run[r]);
        if (g == 0) l_run[r] += p;  // the epilogue sums l over the four lane groups
        const float pw = p * vsf;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(lds + 128 + 16 * d + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[r][d][e] = fmaf(pw, v4[e], acc[r][d][e]);
        }
      }
    }
  };
  auto new_token = [&](int j, float k0, float k1, float v0, float v1, int64_t slot, bool store)
                       __attribute__((always_inline)) {
    uint32_t kw, vw;
    float ks_t, vs_t;
    write_token(k0, k1, v0, v1, slot, store, &kw, &vw, &ks_t, &vs_t);
    fold_token(j, kw, vw, ks_t, vs_t);
  };

  // One-row workgroups: the wave's first new token is quantized and stored
  // now, while the first pages load (its loads were issued first, so the
  // wait is for them alone), and attended after the stream.  Two-row
  // workgroups (two waves per SIMD, registers full) do both after the
  // stream: measured, their step was 0.7 us longer this way.
  constexpr bool kEarlyWrite = RT == 1;
  uint32_t fz_kw = 0, fz_vw = 0;
  float fz_ks = 1.0f, fz_vs = 1.0f;
  if constexpr (FW && kEarlyWrite) {
    if (fz_mine)
      write_token(fk0, fk1, fv0, fv1, fslot, SPARSE ? part == 0 : fz_i0 == 0, &fz_kw, &fz_vw, &fz_ks, &fz_vs);
  }

  // ---- stream the partition's pages: a ring of NBUF chunk buffers, the
  // loads of the next NBUF-1 pages in flight while one is processed.  Table
  // entries are read one step ahead of their use. -------------------------
  if (s0 < n1) {
#pragma unroll
    for (int k = 1; k < NBUF - 1; ++k) {
      const int pos = s0 + k * S;
      const int ln = logical_at(pos);
      const int P = raw_at(pos, ln);
      const bool ok = valid_page(P);
      tb[k] = ok ? ln * 128 : kNoTokens;
      load_chunk<PER_TOKEN, BF, kOnce>(buf[k], a, int64_t(P) * a.hkv + h, ok, lofs);
    }
    // raw entry of the next position to load (s0 + (NBUF-1)*S) and the
    // logical page of the one after it
    int ln_next = logical_at(s0 + (NBUF - 1) * S);
    int P_next = raw_at(s0 + (NBUF - 1) * S, ln_next);
    int ln_after = logical_at(s0 + NBUF * S);
    // Every step of an iteration runs, also past n1 (those positions were
    // loaded as empty and take the skip path): an early exit between steps
    // would leave the next step's loads pending at the loop latch, and the
    // compiler would then wait for the current chunk before issuing the
    // next one -- serializing the ring.
    for (int n = s0; n < n1; n += NBUF * S) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        const int nn = n + k * S;
        const int ls = (k + NBUF - 1) % NBUF;  // slot of position nn + (NBUF-1)*S (held nn - S)
        const int nl = nn + (NBUF - 1) * S;
        const bool ok = valid_page(P_next);
        tb[ls] = ok ? ln_next * 128 : kNoTokens;
        load_chunk<PER_TOKEN, BF, kOnce>(buf[ls], a, int64_t(P_next) * a.hkv + h, ok, lofs);
        // table reads for the following steps (checked one step later)
        ln_next = ln_after;
        P_next = raw_at(nl + S, ln_next);
        ln_after = logical_at(nl + 2 * S);
        process(buf[k], tb[k]);
      }
    }
  }

  if constexpr (FW && SPARSE) {
    // the row's one new token (stored by partition 0 before the stream),
    // attended here if this workgroup's stream passed its page
    if (wave == 0 && fz_seen) fold_token(0, fz_kw, fz_vw, fz_ks, fz_vs);
  } else if constexpr (FW) {
    // row group 0 of the last partition stores each new token once
    if constexpr (kEarlyWrite) {
      if (fz_pend) fold_token(wave, fz_kw, fz_vw, fz_ks, fz_vs);
    } else {
      if (fz_pend) new_token(wave, fk0, fk1, fv0, fv1, fslot, fz_i0 == 0);
    }
    if (fz_last) {
      for (int j = wave + NW; j < fz_L; j += NW) {
        const int64_t t = fz_start + j;
        float k0, k1, v0, v1;
        load_pair(a.k_new, t * a.kn_tok_stride + h * a.kn_head_stride + 2 * lane, a.kn_bf16, &k0, &k1);
        load_pair(a.v_new, t * a.vn_tok_stride + h * a.vn_head_stride + 2 * lane, a.kn_bf16, &v0, &v1);
        new_token(j, k0, k1, v0, v1, a.slots[t], fz_i0 == 0);
      }
    }
  }

  // ---- merge the waves, then write output or the partition partial --------
  // Every wave leaves each row's (max, sum) and unscaled accumulators in
  // LDS; after one barrier, 256 threads per row (a workgroup of 256 takes
  // the rows in turn) weight the waves' accumulators of their (head, 8
  // dims) by 2^(m_w - max) and sum them.
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    if (r >= nrows) break;
    float lh = l_run[r];
    lh += __shfl_xor(lh, 16, kWave);
    lh += __shfl_xor(lh, 32, kWave);
    if (g == 0) {
      sm_ml[wave][r][hr][0] = m_run[r];
      sm_ml[wave][r][hr][1] = lh;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) *reinterpret_cast<f32x4*>(&sm_acc[r][wave][hr][16 * d + 4 * g]) = acc[r][d];
  }
  __syncthreads();
  const int oh = (t >> 4) & 15;  // output head handled by this thread
  const int od = (t & 15) * 8;   // first of its 8 dims
  for (int r = t >> 8; r < nrows; r += (kWave * NW) >> 8) {
    float mw[NW];
    float Mo = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = sm_ml[w][r][oh][0];
      Mo = fmaxf(Mo, mw[w]);
    }
    float Ls = 0.0f;
    f32x4 s0v = {0.f, 0.f, 0.f, 0.f}, s1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      // a wave that saw no token has m = -inf: weight 0
      const float fw = (Mo == -INFINITY || mw[w] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - Mo);
      Ls += fw * sm_ml[w][r][oh][1];
      s0v += fw * *reinterpret_cast<const f32x4*>(&sm_acc[r][w][oh][od]);
      s1v += fw * *reinterpret_cast<const f32x4*>(&sm_acc[r][w][oh][od + 4]);
    }
    const int row = row0 + r;
    const int qh = 16 * h + oh;
    if (!to_partial) {
      const float inv = Ls > 0.0f ? v_fold / Ls : 0.0f;
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        packed[e] = uint32_t(f32_to_bf16_rne(s0v[2 * e] * inv)) |
                    (uint32_t(f32_to_bf16_rne(s0v[2 * e + 1] * inv)) << 16);
        packed[2 + e] = uint32_t(f32_to_bf16_rne(s1v[2 * e] * inv)) |
                        (uint32_t(f32_to_bf16_rne(s1v[2 * e + 1] * inv)) << 16);
      }
      uint16_t* op = a.out + int64_t(row) * a.out_row_stride + int64_t(qh) * a.out_head_stride + od;
      *reinterpret_cast<u32x4*>(op) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    } else {
      const int64_t pi = (prow0 + r) * Hq + qh;
      if (a.unit_count) {
        float* ap = a.part_acc + pi * 128 + od;
        store_coherent(ap, s0v[0], s0v[1]);
        store_coherent(ap + 2, s0v[2], s0v[3]);
        store_coherent(ap + 4, s1v[0], s1v[1]);
        store_coherent(ap + 6, s1v[2], s1v[3]);
        if ((t & 15) == 0) store_coherent(a.part_ml + 2 * pi, Mo, Ls);
      } else {
        f32x4* ap = reinterpret_cast<f32x4*>(a.part_acc + pi * 128 + od);
        ap[0] = s0v;
        ap[1] = s1v;
        if ((t & 15) == 0) {
          a.part_ml[2 * pi] = Mo;
          a.part_ml[2 * pi + 1] = Ls;
        }
      }
    }
  }
  // (merge_if_last starts with a barrier before it reuses the LDS)
  if (a.parts > 1 && a.unit_count) merge_if_last(a, unit, row0, nrows, h, &sm_acc[0][0][0][0]);
}

// One wavefront per (row, query head): combine the partitions' (m, l, acc)
// with log-sum-exp weights and write bf16.  Partitions go in batches of up
// to 64: lane p holds (m, l) of partition p0 + p, so the batch maximum and
// weight sum are cross-lane reductions; every lane owns dims 2*lane,
// 2*lane+1 and takes each partition's weight from its lane.  All loads of a
// batch -- (m, l) and every accumulator -- are issued together, so a batch
// costs one memory round trip; no barrier, no LDS.  N: accumulator loads
// per batch (the partition count rounded up to 8, 16, 32 or 64).
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// One wave's share of a (row, query head): partitions [q0, q1), merged into
// (M, L, ox, oy) relative to its own running maximum M.  Partition p's
// partial is entry p * stride_p + base of the (m, l) and accumulator arrays.
template <int N>
__device__ __forceinline__ void merge_range(const DecodeArgs& a, int64_t base, int64_t stride_p, int q0, int q1,
                                            float& M, float& L, float& ox, float& oy) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int p0 = q0; p0 < q1; p0 += N) {
    const int cnt = min(N, q1 - p0);
    float2 v[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int p = p0 + min(j, cnt - 1);
      v[j] = *reinterpret_cast<const float2*>(a.part_acc + (p * stride_p + base) * 128 + 2 * lane);
    }
    float2 ml = {-INFINITY, 0.0f};
    if (lane < cnt) ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * ((p0 + lane) * stride_p + base));
    const float Mn = fmaxf(M, wave_max(ml.x));
    const float keep = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float w = (ml.x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml.x - Mn);
    L = L * keep + wave_sum(w * ml.y);
    ox *= keep;
    oy *= keep;
    M = Mn;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float wj = lane_value(w, j);
      if (j < cnt && wj != 0.0f) {
        ox += wj * v[j].x;
        oy += wj * v[j].y;
      }
    }
  }
}

// blockDim.x / 64 waves per (row, query head), each merging a contiguous
// share of the partitions in one memory round trip (up to 16 of them);
// the waves' results combine through LDS.
__global__ __launch_bounds__(4 * kWave) void pa_merge(DecodeArgs a) {
  __shared__ float sm_ml[4][2];
  __shared__ float2 sm_o[4][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int Hq = 16 * a.hkv;
  const int64_t pair = blockIdx.x;
  const int row = int(pair / Hq);
  const int qh = int(pair - int64_t(row) * Hq);
  uint16_t* op = a.out + int64_t(row) * a.out_row_stride + int64_t(qh) * a.out_head_stride + 2 * lane;
  int64_t base = int64_t(row) * Hq + qh;
  int64_t stride_p = int64_t(a.rows) * Hq;  // between partitions
  int P = a.parts;
  if (a.balanced) {
    // the row's request and its place in it (with nondecreasing
    // cu_seqlens_q: the request starts after the first at or before the
    // row), then that request's slots
    const Balanced bl = balanced_layout(a);
    int b, i;
    if (a.cu_seqlens_q) {
      const int cu = lane < a.batch ? a.cu_seqlens_q[lane] : 0;
      b = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane >= 1 && lane < a.batch && cu <= row));
      i = row - min(max(lane_int(cu, b), 0), a.rows);
    } else {
      b = row / a.uniform_q_len;
      i = row - b * a.uniform_q_len;
    }
    if (i < 0 || i >= a.lrows) {
      // a row the main kernel has no partial for (more rows in its request
      // than max_q_len, or a malformed cu_seqlens_q): zeros
      if (wave == 0) *reinterpret_cast<uint32_t*>(op) = 0u;
      return;
    }
    P = lane_int(bl.parts, b);
    stride_p = int64_t(a.lrows) * Hq;
    base = (int64_t(lane_int(bl.first, b)) * a.lrows + i) * Hq + qh;
  }
  const int share = (P + nw - 1) / nw;
  const int q0 = min(P, wave * share), q1 = min(P, q0 + share);

  // Every launched partition left a partial; empty ones have m = -inf and
  // weight 0 (their accumulators are never read into the sum).
  float M = -INFINITY, L = 0.0f, ox = 0.0f, oy = 0.0f;
  if (share <= 8) merge_range<8>(a, base, stride_p, q0, q1, M, L, ox, oy);
  else if (share <= 16) merge_range<16>(a, base, stride_p, q0, q1, M, L, ox, oy);
  else merge_range<32>(a, base, stride_p, q0, q1, M, L, ox, oy);
  if (nw > 1) {
    if (lane == 0) {
      sm_ml[wave][0] = M;
      sm_ml[wave][1] = L;
    }
    sm_o[wave][lane] = float2{ox, oy};
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
    for (int w = 0; w < nw; ++w) Mt = fmaxf(Mt, sm_ml[w][0]);
    L = 0.0f;
    ox = oy = 0.0f;
    for (int w = 0; w < nw; ++w) {
      const float f = (sm_ml[w][0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sm_ml[w][0] - Mt);
      if (f != 0.0f) {
        L += f * sm_ml[w][1];
        ox += f * sm_o[w][lane].x;
        oy += f * sm_o[w][lane].y;
      }
    }
  }
  float v_fold = 1.0f;
  if (a.scale_mode != PA_SCALE_PER_TOKEN && a.v_scale) v_fold = *a.v_scale;
  const float inv = L > 0.0f ? v_fold / L : 0.0f;
  const uint32_t packed = uint32_t(f32_to_bf16_rne(ox * inv)) | (uint32_t(f32_to_bf16_rne(oy * inv)) << 16);
  *reinterpret_cast<uint32_t*>(op) = packed;
}

// With events, the dispatch itself records them (start and end of this
// kernel), so the measured time is the kernel's own, without marker packets.
template <int RT, bool PT, bool SP, int NB, int NW, bool BF, bool FW, bool O2>
void launch_main_k(const DecodeArgs& a, int64_t grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (e0 || e1)
    hipExtLaunchKernelGGL((pa_decode_main<RT, PT, SP, NB, NW, BF, FW, O2>), dim3(uint32_t(grid)),
                          dim3(kWave * NW), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((pa_decode_main<RT, PT, SP, NB, NW, BF, FW, O2>), dim3(uint32_t(grid)), dim3(kWave * NW),
                       0, s, a);
}

// two-row shapes: the non-temporal instance where at most two row groups
// read each page
template <int RT, bool PT, bool SP, int NB, int NW, bool BF, bool FW = false>
void launch_main_t(const DecodeArgs& a, int64_t grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if constexpr (RT == 2) {
    if (a.kv_once) return launch_main_k<RT, PT, SP, NB, NW, BF, FW, true>(a, grid, s, e0, e1);
  }
  launch_main_k<RT, PT, SP, NB, NW, BF, FW, false>(a, grid, s, e0, e1);
}

// prefetch depth and workgroup width: eight waves (two pages side by side)
// use the two-page ring; deeper rings are a four-wave tuning option.
// A bf16 cache (twice the bytes per chunk) always uses the two-page ring,
// and four waves when a workgroup carries two rows.
template <int RT, bool PT, bool SP, bool BF = false>
void launch_shape(const DecodeArgs& a, int depth, int waves, int64_t grid, hipStream_t s, hipEvent_t e0,
                  hipEvent_t e1) {
  if constexpr (SP) {
    // the sparse fused write (single-row requests): four waves, the two-page ring
    if (a.fused) return launch_main_t<1, PT, true, 2, 4, BF, true>(a, grid, s, e0, e1);
  } else {
    // the fused write: the two-page ring at either width (two-row bf16: four waves)
    if (a.fused) {
      if constexpr (!(BF && RT == 2)) {
        if (waves == 8) return launch_main_t<RT, PT, SP, 2, 8, BF, true>(a, grid, s, e0, e1);
      }
      return launch_main_t<RT, PT, SP, 2, 4, BF, true>(a, grid, s, e0, e1);
    }
  }
  if constexpr (BF && RT == 2) {
    launch_main_t<RT, PT, SP, 2, 4, BF>(a, grid, s, e0, e1);
  } else {
    if (waves == 8) return launch_main_t<RT, PT, SP, 2, 8, BF>(a, grid, s, e0, e1);
    if constexpr (!SP && !BF) {
      if (depth == 3) return launch_main_t<RT, PT, SP, 3, 4, BF>(a, grid, s, e0, e1);
      if (depth >= 4) return launch_main_t<RT, PT, SP, 4, 4, BF>(a, grid, s, e0, e1);
    }
    launch_main_t<RT, PT, SP, 2, 4, BF>(a, grid, s, e0, e1);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int64_t grid, bool merge, bool sparse, int depth, int waves,
                         hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const bool pt = a.scale_mode == PA_SCALE_PER_TOKEN;
  hipEvent_t e0 = ev_begin, e1 = ev_end;
  // the one variant-selection table: (cache element type, rows per group,
  // per-token scales, sparse, prefetch depth, waves per workgroup)
  const int d = depth, w = waves;
  if (a.prefill) {
    hipError_t pe = launch_prefill_main(a, grid, e0, e1, stream);
    if (pe != hipSuccess) return pe;
  } else if (a.kv_bf16) {
    // unquantized cache: never scaled
    if (sparse) launch_shape<1, false, true, true>(a, d, w, grid, stream, e0, e1);
    else if (a.rt == 1) launch_shape<1, false, false, true>(a, d, w, grid, stream, e0, e1);
    else launch_shape<2, false, false, true>(a, d, w, grid, stream, e0, e1);
  } else if (sparse) {
    if (pt) launch_shape<1, true, true>(a, d, w, grid, stream, e0, e1);
    else launch_shape<1, false, true>(a, d, w, grid, stream, e0, e1);
  } else if (a.rt == 1) {
    if (pt) launch_shape<1, true, false>(a, d, w, grid, stream, e0, e1);
    else launch_shape<1, false, false>(a, d, w, grid, stream, e0, e1);
  } else {
    if (pt) launch_shape<2, true, false>(a, d, w, grid, stream, e0, e1);
    else launch_shape<2, false, false>(a, d, w, grid, stream, e0, e1);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (merge && !a.unit_count) {
    const int64_t pairs = int64_t(a.rows) * 16 * a.hkv;
    // one wave per 16 partitions, at most four.  Balanced: a request's
    // partition count is known only on the device and is usually a few, so
    // one wave, which takes any count in batches of up to 32 (measured at
    // q_len 4: four waves that each derive the split cost 12 us, one 4.6)
    const int waves = a.balanced ? 1 : (a.parts <= 16 ? 1 : (a.parts <= 32 ? 2 : 4));
    hipLaunchKernelGGL(pa_merge, dim3(uint32_t(pairs)), dim3(kWave * waves), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace fp8pa
