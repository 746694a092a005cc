// Device-side check of a decode call's inputs: the preconditions pa_decode
// documents but cannot verify on the host without reading device memory
// (ROCm/ATOM pull request 2122, section 2: a decode segment's row layout
// must match what the kernel assumes, and the kernel-side check stays as a
// backstop).  Here the check is its own launch that writes a report instead
// of trapping.
//
// Report (int32[16], see pa_check_kind): [0] violating items, [1] bitmask of
// kinds, [2 + k] smallest offending index of kind k (INT32_MAX if none).
//
// Grid: workgroups [0, batch) take one request each -- cu_seqlens_q ends and
// order, context length against q_len, and (dense calls) the block-table
// ids and per-token scales of every attended page; workgroups
// [batch, batch + rows) of a sparse call take one query row each -- list
// entries, duplicates, and the table ids and scales of the listed pages the
// row sees.  Every read is bounded by the descriptors' sizes, never by a
// device value alone.
#include <climits>

#include "device_common.h"
#include "check.h"

namespace fp8pa {

namespace {

constexpr int kCheckThreads = 256;
constexpr int kKinds = 7;

// One thread's findings, folded into the report once at the end.
struct Found {
  int count = 0;
  int mask = 0;
  int first[kKinds];
  __device__ Found() {
    for (int k = 0; k < kKinds; ++k) first[k] = INT_MAX;
  }
  __device__ void add(int kind, int64_t index) {
    ++count;
    mask |= 1 << kind;
    const int i = index > INT_MAX ? INT_MAX : int(index);
    first[kind] = min(first[kind], i);
  }
};

__device__ __forceinline__ bool finite_bits(float x) {
  return (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u;
}

// Per-token K and V scales of one (head, slot) of physical page P, logical
// page n of request b.
__device__ __forceinline__ void check_scale(const DecodeArgs& a, int b, int n, int64_t P, int h, int o, Found& f) {
  const int64_t si = (P * a.hkv + h) * 128 + o;
  const float ks = a.k_scale[si], vs = a.v_scale[si];
  if (!finite_bits(ks) || !finite_bits(vs) || ks < 0.0f || vs < 0.0f) f.add(6, int64_t(b) * a.width + n);
}

// Request b's rows [start, start + L) with L >= 0; cu_seqlens_q values are
// clamped into [0, rows] as the decode kernel clamps them.
__device__ __forceinline__ void rows_of(const DecodeArgs& a, int b, int* start, int* L) {
  if (a.cu_seqlens_q) {
    const int s = min(max(a.cu_seqlens_q[b], 0), a.rows);
    const int e = min(max(a.cu_seqlens_q[b + 1], s), a.rows);
    *start = s;
    *L = e - s;
  } else {
    *L = a.uniform_q_len;
    *start = b * a.uniform_q_len;
  }
}

__global__ __launch_bounds__(kCheckThreads) void check_init_kernel(int32_t* report) {
  const int t = threadIdx.x;
  if (t < 16) report[t] = t < 2 ? 0 : INT_MAX;
}

__global__ __launch_bounds__(kCheckThreads) void check_kernel(DecodeArgs a, int32_t* report) {
  Found f;
  const int64_t wg = blockIdx.x;
  const bool per_token = a.scale_mode == PA_SCALE_PER_TOKEN && !a.kv_bf16;
  if (wg < a.batch) {
    const int b = int(wg);
    if (threadIdx.x == 0) {
      if (a.cu_seqlens_q) {
        if (b == 0 && (a.cu_seqlens_q[0] != 0 || a.cu_seqlens_q[a.batch] != a.rows)) f.add(0, 0);
        if (a.cu_seqlens_q[b + 1] < a.cu_seqlens_q[b]) f.add(1, b);
      }
      int start, L;
      rows_of(a, b, &start, &L);
      if (a.context_lens[b] < L) f.add(2, b);
      if (b == 0 && a.scale_mode == PA_SCALE_SCALAR) {
        const float ks = *a.k_scale, vs = *a.v_scale;
        if (!finite_bits(ks) || !finite_bits(vs) || !(ks > 0.0f) || !(vs > 0.0f)) f.add(6, 0);
      }
    }
    if (!a.sparse_idx) {
      // dense: every page the request's last row sees
      const int limit = max(0, min(a.context_lens[b], a.width * 128));
      const int npages = (limit + 127) >> 7;
      const int32_t* bt = a.block_table + int64_t(b) * a.bt_stride;
      for (int n = threadIdx.x; n < npages; n += kCheckThreads)
        if (bt[n] < 0 || bt[n] >= a.num_blocks) f.add(3, int64_t(b) * a.width + n);
      if (per_token) {
        // every (page, head, slot) of the attended tokens, spread over the threads
        const int per_page = a.hkv * 128;
        const int64_t total = int64_t(npages) * per_page;
        for (int64_t i = threadIdx.x; i < total; i += kCheckThreads) {
          const int n = int(i / per_page), r = int(i - int64_t(n) * per_page);
          const int h = r >> 7, o = r & 127;
          const int64_t P = bt[n];
          if (n * 128 + o < limit && P >= 0 && P < a.num_blocks) check_scale(a, b, n, P, h, o, f);
        }
      }
    }
  } else if (a.sparse_idx && wg < int64_t(a.batch) + a.rows) {
    const int row = int(wg - a.batch);
    // the row's request: the one whose row range holds it (request 0 when
    // none does, as with a malformed cu_seqlens_q -- reported above)
    int b = 0, start = 0, L = 0;
    if (a.cu_seqlens_q) {
      for (int j = 0; j < a.batch; ++j) {
        int s, l;
        rows_of(a, j, &s, &l);
        if (s <= row && row < s + l) {
          b = j;
          start = s;
          L = l;
        }
      }
    } else {
      b = row / a.uniform_q_len;
      rows_of(a, b, &start, &L);
    }
    const int limit = max(0, min(a.context_lens[b] - L + (row - start) + 1, a.width * 128));
    const int32_t* list = a.sparse_idx + int64_t(row) * a.sp_stride;
    const int32_t* bt = a.block_table + int64_t(b) * a.bt_stride;
    for (int i = threadIdx.x; i < a.topk; i += kCheckThreads) {
      const int n = list[i];
      if (n == -1) continue;
      if (n < 0 || n >= a.width) {
        f.add(4, int64_t(row) * a.topk + i);
        continue;
      }
      for (int j = i + 1; j < a.topk; ++j)
        if (list[j] == n) {
          f.add(5, row);
          break;
        }
      if (n * 128 < limit && (bt[n] < 0 || bt[n] >= a.num_blocks)) f.add(3, int64_t(b) * a.width + n);
    }
    if (per_token) {
      // every (list entry, head, slot) of the tokens the row sees
      const int per_page = a.hkv * 128;
      const int64_t total = int64_t(a.topk) * per_page;
      for (int64_t i = threadIdx.x; i < total; i += kCheckThreads) {
        const int e = int(i / per_page), r = int(i - int64_t(e) * per_page);
        const int h = r >> 7, o = r & 127;
        const int n = list[e];
        if (n < 0 || n >= a.width || n * 128 + o >= limit) continue;
        const int64_t P = bt[n];
        if (P >= 0 && P < a.num_blocks) check_scale(a, b, n, P, h, o, f);
      }
    }
  }
  if (f.count) {
    atomicAdd(report, f.count);
    atomicOr(report + 1, f.mask);
    for (int k = 0; k < kKinds; ++k)
      if (f.mask & (1 << k)) atomicMin(report + 2 + k, f.first[k]);
  }
}

}  // namespace

hipError_t launch_check(const DecodeArgs& a, int32_t* report, hipStream_t stream) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(kCheckThreads), 0, stream, report);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t grid = int64_t(a.batch) + (a.sparse_idx ? a.rows : 0);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(check_kernel, dim3(uint32_t(grid)), dim3(kCheckThreads), 0, stream, a, report);
  return hipGetLastError();
}

}  // namespace fp8pa
