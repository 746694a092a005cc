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
// tile tau reads the 32 contiguous bytes of dims 32g..32g+31 of token
// 16*tau + r; k-step j takes dims 32g + 8j .. +7 of that run, and the query
// operand takes the same dims, so the dot product is over every dim once.
//
// index_topk_kernel: one workgroup per row.  A four-pass, 8-bit radix
// select finds the k-th largest score (scores mapped to order-preserving
// unsigned keys); a block-wide scan then writes the chosen pages in
// ascending order, taking ties at the threshold from the lowest page up.
#include "device_common.h"
#include "launch.h"

namespace fp8pa {

namespace {

constexpr int kIdxWaves = 4;     // pages per score workgroup (one per wave)
constexpr int kTopkThreads = 256;  // one thread per radix bin in the digit search
constexpr int kStageKeys = 8192;   // rows with up to this many pages keep their keys in LDS

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

  // K: token 16*tau + r, dims 32g .. 32g+31 (two 16-byte loads per tile)
  const uint8_t* kp = a.index_cache + int64_t(P) * 16384 + r * 128 + 32 * g;
  u32x4 kb[8][2];
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    kb[tau][0] = *reinterpret_cast<const u32x4*>(kp + tau * 2048);
    kb[tau][1] = *reinterpret_cast<const u32x4*>(kp + tau * 2048 + 16);
  }
  // Q^T operand: column r = row i0 + r, dims 32g + 8j .. +7 for k-step j
  bf16x8 qop[4];
  if (r < nrows) {
    const uint16_t* qp = a.q + int64_t(start + i0 + r) * a.q_row_stride + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) qop[j] = *reinterpret_cast<const bf16x8*>(qp + 8 * j);
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

// Block-wide exclusive scan of one value per thread (kTopkThreads threads);
// also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* sm_wave) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  if (lane == kWave - 1) sm_wave[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    const int s = sm_wave[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

__global__ __launch_bounds__(kTopkThreads) void index_topk_kernel(IndexArgs a) {
  __shared__ int hist[256];
  __shared__ int sm_wave[kTopkThreads / kWave];
  __shared__ uint32_t sm_sel[2];  // threshold digit result, remaining count
  __shared__ uint32_t sm_keys[kStageKeys];
  const int row = blockIdx.x;
  const int t = threadIdx.x;

  // the request of this row and its visible page count
  int b, start, L;
  if (a.cu_seqlens_q) {
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid;
    }
    b = lo;
    start = min(max(a.cu_seqlens_q[b], 0), a.rows);
    L = min(max(a.cu_seqlens_q[b + 1], start), a.rows) - start;
  } else {
    L = a.uniform_q_len;
    b = row / L;
    start = b * L;
  }
  const int lim = max(0, min(a.context_lens[b] - L + (row - start) + 1, a.width * 128));
  const int n = (lim + 127) >> 7;  // pages the row can see
  const float* srow = a.scores + int64_t(row) * a.score_stride;
  int32_t* orow = a.out_idx + int64_t(row) * a.out_stride;
  const int k = a.topk;

  // keys of the row: staged once in LDS (coalesced read) when they fit,
  // else read from the score matrix on every pass
  const bool staged = n <= kStageKeys;
  if (staged) {
    for (int i = t; i < n; i += kTopkThreads) sm_keys[i] = score_key(srow[i]);
    __syncthreads();
  }
  auto key_at = [&](int i) -> uint32_t { return staged ? sm_keys[i] : score_key(srow[i]); };

  // this thread's contiguous slice of the row's pages
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int c0 = min(n, t * chunk), c1 = min(n, c0 + chunk);

  int fin = 0;
  for (int i = c0; i < c1; ++i) fin += key_at(i) != 0u;
  int total_fin;
  block_exclusive_scan(fin, &total_fin, sm_wave);

  uint32_t thr = 1u;  // keys >= thr are candidates; 1 keeps every finite score
  int need_eq = 0;    // ties at the threshold still to take (lowest pages first)
  if (total_fin > k) {
    uint32_t prefix = 0, mask = 0;
    int rem = k;
    for (int d = 3; d >= 0; --d) {
      const int sh = 8 * d;
      for (int i = t; i < 256; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
      for (int i = c0; i < c1; ++i) {
        const uint32_t key = key_at(i);
        if (key != 0u && (key & mask) == prefix) atomicAdd(&hist[(key >> sh) & 255u], 1);
      }
      __syncthreads();
      // the digit D with count(digit > D) < rem <= count(digit >= D): thread
      // t holds digit 255 - t, an exclusive scan gives count(digit > D)
      {
        const int D = 255 - t;
        const int cnt = hist[D];
        int tot;
        const int above = block_exclusive_scan(cnt, &tot, sm_wave);
        if (above < rem && rem <= above + cnt) {
          sm_sel[0] = uint32_t(D);
          sm_sel[1] = uint32_t(rem - above);
        }
      }
      __syncthreads();
      prefix |= sm_sel[0] << sh;
      mask |= 255u << sh;
      rem = int(sm_sel[1]);
      __syncthreads();
    }
    thr = prefix;  // the k-th largest key; rem of the keys equal to it are taken
    need_eq = rem;
  }

  // pass 1: counts; pass 2: write the chosen pages in ascending order
  int gt = 0, eq = 0;
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = key_at(i);
    if (total_fin > k) {
      gt += key > thr;
      eq += key == thr;
    } else {
      gt += key != 0u;
    }
  }
  int dummy;
  const int eq_before = block_exclusive_scan(eq, &dummy, sm_wave);
  const int take_eq = total_fin > k ? min(max(need_eq - eq_before, 0), eq) : 0;
  int total_sel;
  int pos = block_exclusive_scan(gt + take_eq, &total_sel, sm_wave);
  int eq_left = take_eq;
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = key_at(i);
    bool pick;
    if (total_fin > k) {
      pick = key > thr || (key == thr && eq_left > 0);
      if (key == thr && eq_left > 0) --eq_left;
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
