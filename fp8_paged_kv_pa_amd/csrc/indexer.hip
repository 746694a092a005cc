// Sparse indexer: block scores over the fp8 index cache, then the per-row
// top-k of logical pages that the block-sparse decode attends.
//
// What is computed (ROCm/ATOM pull request 2122, "fix(minimax-m3): unblock
// fp8 KV cache and EAGLE3 spec decode on the vLLM plugin": section 1 --
// the index cache is float8_e4m3fn (num_blocks, 128, 128) and the block
// score is the fp32 product of the index query with the fp8 keys times
// sm_scale * log2(e); section 2 -- row i of a q_len-L request has the
// causal cutoff ctx - L + i + 1):
//   s_t      = sm_scale * log2(e) * <q_row, k_t>          (visible tokens t)
//   score_n  = log2 sum_{t in page n} 2^(s_t)              (-inf if none)
//   list_row = the topk highest finite scores, ties to the lower page,
//              in ascending page order, padded with -1.
//
// index_score_kernel: one wave per (request, group of up to 16 rows,
// logical page).  The rows of the group are the 16 columns of
//   S^T[token, row] = K[token, d] * Q^T[d, row]   (bf16 MFMA 16x16x32)
// so the 16 KiB page is read once for all rows of a request (q_len 4 uses
// 4 of the columns).  Index keys are token-major, so lane (r, g) of token
// tile tau reads dims 16g..16g+15 and 64+16g..64+16g+15 of token 16*tau + r
// (each of the two load instructions then covers whole 64-byte runs of the
// tile); k-step j takes dims 64(j/2) + 16g + 8(j%2) .. +7, and the query
// operand takes the same dims, so the dot product is over every dim once.
//
// index_topk_kernel: one workgroup per row.  Scores are mapped to
// order-preserving unsigned keys; bytes that all finite keys of the row
// share are skipped, and an 8-bit radix select over the rest finds the k-th
// largest (LDS histograms, the digit search by one wave, two barriers per
// byte); once at most 64 keys share the bytes chosen so far, one wave ranks
// those few directly.  A block-wide scan then writes the chosen pages in ascending
// order, taking ties at the threshold from the lowest page up.
#include "device_common.h"
#include "launch.h"

namespace fp8pa {

namespace {

constexpr int kIdxWaves = 4;     // pages per score workgroup (one per wave)
constexpr int kTopkThreads = 256;  // one histogram entry per thread
constexpr int kStageKeys = 8192;   // rows with up to this many pages keep their keys in LDS
constexpr int kLoadBatch = 8;      // key loads a thread issues before using them

typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
__device__ __forceinline__ const_i32_ptr as_const(const int32_t* p) { return (const_i32_ptr)(p); }

__global__ __launch_bounds__(kWave * kIdxWaves) void index_score_kernel(IndexArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int r = lane & 15;  // token within a 16-token tile / column (row) of the group
  const int g = lane >> 4;  // 32-dim slice of the index key
  const int64_t pblocks = (int64_t(a.width) + kIdxWaves - 1) / kIdxWaves;
  const int64_t unit = blockIdx.x / pblocks;
  const int n = int(blockIdx.x - unit * pblocks) * kIdxWaves + wave;  // logical page
  if (n >= a.width) return;
  const int gi = int(unit % a.groups);
  const int b = int(unit / a.groups);

  int start, L;
  if (a.cu_seqlens_q) {
    start = min(max(a.cu_seqlens_q[b], 0), a.rows);
    L = min(max(a.cu_seqlens_q[b + 1], start), a.rows) - start;
  } else {
    L = a.uniform_q_len;
    start = b * L;
  }
  const int i0 = 16 * gi;
  if (i0 >= L) return;
  const int nrows = min(16, L - i0);
  const int ctx = a.context_lens[b];
  const int cap = a.width * 128;
  // this lane's column: row i0 + r of the request (when r < nrows)
  const int lim_r = max(0, min(ctx - L + i0 + r + 1, cap));
  const int lim_max = max(0, min(ctx - L + i0 + nrows, cap));

  float* srow = a.scores + int64_t(start + i0 + r) * a.score_stride;
  if (n * 128 >= lim_max) {
    // no row of the group sees this page
    if (g == 0 && r < nrows) srow[n] = -INFINITY;
    return;
  }
  const int P = as_const(a.block_table + int64_t(b) * a.bt_stride)[n];
  if (P < 0 || P >= a.num_blocks) {
    if (g == 0 && r < nrows) srow[n] = -INFINITY;
    return;
  }

  // K: token 16*tau + r, dims 16g .. 16g+15 and 64+16g .. 64+16g+15 (two
  // 16-byte loads per tile; each load instruction covers whole 64-byte
  // runs, one per token)
  const uint8_t* kp = a.index_cache + int64_t(P) * 16384 + r * 128 + 16 * g;
  u32x4 kb[8][2];
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    kb[tau][0] = *reinterpret_cast<const u32x4*>(kp + tau * 2048);
    kb[tau][1] = *reinterpret_cast<const u32x4*>(kp + tau * 2048 + 64);
  }
  // Q^T operand: column r = row i0 + r, the same dims as K for each k-step:
  // k-step j takes dims 64(j/2) + 16g + 8(j%2) .. +7
  bf16x8 qop[4];
  if (r < nrows) {
    const uint16_t* qp = a.q + int64_t(start + i0 + r) * a.q_row_stride + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) qop[j] = *reinterpret_cast<const bf16x8*>(qp + 64 * (j >> 1) + 8 * (j & 1));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) qop[j] = bf16x8{};
  }

  // S^T for the 8 token tiles; lane (r, g) gets tokens 16*tau + 4g + v of column r
  float m = -INFINITY;
  float x[8][4];
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4& w = kb[tau][j >> 1];
      const bf16x8 kop = fp8x8_to_bf16x8(w[2 * (j & 1)], w[2 * (j & 1) + 1]);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[j], st, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = n * 128 + 16 * tau + 4 * g + v;
      // select, not arithmetic: a masked token's (possibly NaN) product is dropped
      x[tau][v] = t < lim_r ? st[v] * a.sm_log2 : -INFINITY;
      m = fmaxf(m, x[tau][v]);
    }
  }
  // column max and sum over the 4 lane groups holding the same column
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  float sum = 0.0f;
  if (m != -INFINITY) {
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v) sum += __builtin_amdgcn_exp2f(x[tau][v] - m);
  }
  sum += __shfl_xor(sum, 16, kWave);
  sum += __shfl_xor(sum, 32, kWave);
  if (g == 0 && r < nrows) srow[n] = m == -INFINITY ? -INFINITY : m + __log2f(sum);
}

// Order-preserving map of a float score to an unsigned key; -inf (no
// visible token) maps to 0, below every finite score's key.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == -INFINITY) return 0u;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One histogram increment per active lane with act set.  The lanes that
// share the first such lane's bin add their count with one atomic (the
// common case in the leading digits, where a row's keys crowd into a few
// bins); the others add one each.
__device__ __forceinline__ void add_to_bin(int* hist, bool act, uint32_t bin) {
  const uint64_t am = __builtin_amdgcn_ballot_w64(act);
  if (am == 0) return;
  const int leader = __builtin_ctzll(am);
  const uint32_t lb = uint32_t(__builtin_amdgcn_readlane(int(bin), leader));
  const uint64_t same = __builtin_amdgcn_ballot_w64(act && bin == lb);
  if (!act) return;
  if (bin != lb) atomicAdd(&hist[bin], 1);
  else if (int(threadIdx.x & (kWave - 1)) == leader) atomicAdd(&hist[lb], __builtin_popcountll(same));
}

__global__ __launch_bounds__(kTopkThreads) void index_topk_kernel(IndexArgs a) {
  static_assert(kTopkThreads == 4 * kWave, "one histogram entry per thread, digit search by wave 0");
  __shared__ __align__(16) int hist[2][256];  // double-buffered digit histograms
  __shared__ uint32_t sm_stat[3][kTopkThreads / kWave];  // per wave: finite count, max key, min finite key
  __shared__ uint32_t sm_sel[3];              // chosen digit, keys still to take at it, keys with it
  __shared__ uint32_t sm_cand[kWave];         // the last few candidate keys
  __shared__ int sm_ncand;
  __shared__ int sm_scan[2][kTopkThreads / kWave];
  __shared__ uint32_t sm_keys[kStageKeys];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t >> 6;

  const float* srow = a.scores + int64_t(row) * a.score_stride;
  int32_t* orow = a.out_idx + int64_t(row) * a.out_stride;
  const int k = a.topk;

  // the first batch of the row's scores, requested before the row's length
  // is known (every entry below the table width is inside the matrix), so
  // its latency overlaps the request lookup
  float first[kLoadBatch];
#pragma unroll
  for (int j = 0; j < kLoadBatch; ++j) {
    const int i = j * kTopkThreads + t;
    first[j] = i < a.width ? srow[i] : -INFINITY;
  }

  // the request of this row (cu_seqlens_q nondecreasing: the last request
  // starting at or before the row) and its visible page count.  Up to 64
  // requests one load round trip: each wave counts the later starts at or
  // before the row with a ballot; beyond that a binary search.
  int b, start, L;
  if (a.cu_seqlens_q) {
    if (a.batch <= kWave) {
      b = __builtin_popcountll(
          __builtin_amdgcn_ballot_w64(lane >= 1 && lane < a.batch && a.cu_seqlens_q[lane] <= row));
    } else {
      int lo = 0, hi = a.batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid;
      }
      b = lo;
    }
    start = min(max(a.cu_seqlens_q[b], 0), a.rows);
    L = min(max(a.cu_seqlens_q[b + 1], start), a.rows) - start;
  } else {
    L = a.uniform_q_len;
    b = row / L;
    start = b * L;
  }
  const int lim = max(0, min(a.context_lens[b] - L + (row - start) + 1, a.width * 128));
  const int n = (lim + 127) >> 7;  // pages the row can see

  // one coalesced pass over the row: keys staged in LDS when they fit (else
  // read from the score matrix on every pass), the finite count and the
  // range of the finite keys
  const bool staged = n <= kStageKeys;
  // fn(i, key) for pages i = from + t, from + t + 256, ...  From LDS one
  // page at a time; from the score matrix in batches of kLoadBatch loads
  // issued together (one load latency per batch, not per page), where past
  // the row's end fn sees key 0, the key of -inf
  auto for_keys = [&](int from, bool from_lds, auto&& fn) {
    if (from_lds) {
      for (int i = from + t; i < n; i += kTopkThreads) fn(i, sm_keys[i]);
      return;
    }
    for (int base = from; base < n; base += kLoadBatch * kTopkThreads) {
      uint32_t kk[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) {
        const int i = base + j * kTopkThreads + t;
        kk[j] = i < n ? score_key(srow[i]) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) fn(base + j * kTopkThreads + t, kk[j]);
    }
  };
  uint32_t fin = 0u, khi = 0u, klo = 0xFFFFFFFFu;
  auto stage = [&](int i, uint32_t key) {
    if (staged && i < n) sm_keys[i] = key;
    fin += key != 0u;
    khi = max(khi, key);
    klo = min(klo, key ? key : 0xFFFFFFFFu);
  };
#pragma unroll
  for (int j = 0; j < kLoadBatch; ++j) {
    const int i = j * kTopkThreads + t;
    stage(i, i < n ? score_key(first[j]) : 0u);
  }
  for_keys(kLoadBatch * kTopkThreads, false, stage);
  auto key_at = [&](int i) -> uint32_t { return staged ? sm_keys[i] : score_key(srow[i]); };
  hist[0][t] = 0;
  hist[1][t] = 0;
  if (t == 0) sm_ncand = 0;
  fin = wave_reduce_u32<UOp::ADD>(fin);
  khi = wave_reduce_u32<UOp::MAX>(khi);
  klo = wave_reduce_u32<UOp::MIN>(klo);
  if (lane == 0) {
    sm_stat[0][wave] = fin;
    sm_stat[1][wave] = khi;
    sm_stat[2][wave] = klo;
  }
  __syncthreads();
  int total_fin = 0;
  khi = 0u;
  klo = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    total_fin += int(sm_stat[0][w]);
    khi = max(khi, sm_stat[1][w]);
    klo = min(klo, sm_stat[2][w]);
  }

  // the k-th largest key (thr) and how many keys equal to it are taken;
  // without a selection every finite key is taken
  const bool select = total_fin > k;
  uint32_t thr = 1u;
  int need_eq = 0;
  if (select) {
    const uint32_t diff = khi ^ klo;
    if (diff == 0u) {  // every finite key is the same
      thr = khi;
      need_eq = k;
    } else {
      // bytes above the highest byte in which the finite keys differ are
      // the same in all of them, the k-th largest included: take them as
      // they are, and radix-select the rest a byte at a time
      int d = (31 - __builtin_clz(diff)) >> 3;
      uint32_t mask = d == 3 ? 0u : 0xFFFFFFFFu << (8 * (d + 1));
      uint32_t prefix = khi & mask;
      int rem = k, buf = 0;
      for (; d >= 0; --d, buf ^= 1) {
        const int sh = 8 * d;
        for_keys(0, staged, [&](int, uint32_t key) {
          add_to_bin(hist[buf], key != 0u && (key & mask) == prefix, (key >> sh) & 255u);
        });
        // the other buffer serves the next digit; its last reader (wave 0's
        // search of the previous digit) finished before the last barrier
        hist[buf ^ 1][t] = 0;
        __syncthreads();
        if (wave == 0) {
          // lane l holds digits 255-4l down to 252-4l; the digit D with
          // count(digit > D) < rem <= count(digit >= D) is unique
          const int4 c = *reinterpret_cast<const int4*>(&hist[buf][4 * (kWave - 1 - lane)]);
          const int own = c.x + c.y + c.z + c.w;
          int acc = wave_inclusive_scan(own) - own;
          const int cnt[4] = {c.w, c.z, c.y, c.x};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (acc < rem && rem <= acc + cnt[j]) {
              sm_sel[0] = uint32_t(255 - 4 * lane - j);
              sm_sel[1] = uint32_t(rem - acc);
              sm_sel[2] = uint32_t(cnt[j]);
            }
            acc += cnt[j];
          }
        }
        __syncthreads();
        prefix |= sm_sel[0] << sh;
        mask |= 255u << sh;
        rem = int(sm_sel[1]);
        const int few = int(sm_sel[2]);
        if (d > 0 && few <= kWave) {
          // at most 64 keys still share the prefix: gather them and let
          // wave 0 rank them (keys above each, keys equal to it) instead
          // of resolving the remaining bytes
          for_keys(0, staged, [&](int, uint32_t key) {
            if (key != 0u && (key & mask) == prefix) {
              const int slot = atomicAdd(&sm_ncand, 1);
              if (slot < kWave) sm_cand[slot] = key;
            }
          });
          __syncthreads();
          if (wave == 0) {
            const int m = min(sm_ncand, kWave);
            const uint32_t c = lane < m ? sm_cand[lane] : 0u;
            int above = 0, same = 0;
            for (int j = 0; j < m; ++j) {
              const uint32_t cj = uint32_t(__builtin_amdgcn_readlane(int(c), j));
              above += cj > c;
              same += cj == c;
            }
            const bool hit = lane < m && above < rem && rem <= above + same;
            const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
            if (hm != 0 && lane == __builtin_ctzll(hm)) {
              sm_sel[0] = c;
              sm_sel[1] = uint32_t(rem - above);
            }
          }
          __syncthreads();
          prefix = sm_sel[0];
          rem = int(sm_sel[1]);
          break;
        }
      }
      thr = prefix;
      need_eq = rem;
    }
  }

  // each thread's contiguous slice of the row: counts, one block scan of
  // (keys above thr, keys at thr), then the chosen pages
  // in ascending order; ties at thr go to the lowest pages, so the ties
  // taken before a slice number min(need_eq, ties before it)
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int c0 = min(n, t * chunk), c1 = min(n, c0 + chunk);
  int gt = 0, eq = 0;
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = key_at(i);
    if (select) {
      gt += key > thr;
      eq += key == thr;
    } else {
      gt += key != 0u;
    }
  }
  const int gt_inc = wave_inclusive_scan(gt), eq_inc = wave_inclusive_scan(eq);
  if (lane == kWave - 1) {
    sm_scan[0][wave] = gt_inc;
    sm_scan[1][wave] = eq_inc;
  }
  __syncthreads();
  int gt_before = gt_inc - gt, eq_before = eq_inc - eq, gt_tot = 0, eq_tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    const int g = sm_scan[0][w], e = sm_scan[1][w];
    if (w < wave) {
      gt_before += g;
      eq_before += e;
    }
    gt_tot += g;
    eq_tot += e;
  }
  int pos = gt_before + min(need_eq, eq_before);
  const int total_sel = gt_tot + min(need_eq, eq_tot);
  int eq_left = min(max(need_eq - eq_before, 0), eq);
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = key_at(i);
    bool pick;
    if (select) {
      const bool tie = key == thr && eq_left > 0;
      pick = key > thr || tie;
      eq_left -= tie;
    } else {
      pick = key != 0u;
    }
    if (pick) orow[pos++] = i;
  }
  for (int i = total_sel + t; i < k; i += kTopkThreads) orow[i] = -1;
}

}  // namespace

hipError_t launch_index(const IndexArgs& a, int64_t score_grid, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  if (score_grid > 0) {
    hipLaunchKernelGGL(index_score_kernel, dim3(uint32_t(score_grid)), dim3(kWave * kIdxWaves), 0, stream,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(index_topk_kernel, dim3(uint32_t(a.rows)), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

int64_t index_score_grid(int64_t units, int32_t width) {
  return units * ((int64_t(width) + kIdxWaves - 1) / kIdxWaves);
}

}  // namespace fp8pa
