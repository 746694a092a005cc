// C-ABI entry points: descriptor checks (all before any launch), the
// capacity-bucketed split-K scratch, and the kernel launches.
//
// Every condition the host can check is refused with a status code before
// anything runs on the device (ROCm/ATOM pull request 2710 review, "Should
// fix" 2; ROCm/ATOM pull request 2614, "Change": decline a call before the
// low-level launcher would abort).  Scratch comes from one arena per
// (device, stream), sized by capacity bucket and grown only outside graph
// capture (ROCm/ATOM pull request 2710 review, "Must fix" 1: bounded plan
// and scratch shapes, allocated where the memory accounting can see them).
// A replaced arena stays allocated until pa_release, since a graph captured
// with it keeps its address.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/fp8pa.h"
#include "check.h"
#include "launch.h"
#include "plan.h"

namespace fp8pa {
namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int64_t numel(const pa_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

bool contiguous(const pa_tensor* t) {
  int64_t s = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != s) return false;
    s *= t->shape[i];
  }
  return true;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int check_tensor(const pa_tensor* t, const char* name) {
  if (!t) return fail(PA_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (t->ndim < 1 || t->ndim > PA_MAX_DIMS)
    return fail(PA_ERR_SHAPE, std::string(name) + ": ndim out of range");
  for (int i = 0; i < t->ndim; ++i)
    if (t->shape[i] < 0) return fail(PA_ERR_SHAPE, std::string(name) + ": negative extent");
  if (numel(t) > 0 && !t->data) return fail(PA_ERR_INVALID_ARG, std::string(name) + ": data is NULL");
  return PA_OK;
}

// K or V cache: [num_blocks, Hkv, ...] with 16384 elements per (block,
// head) -- FP8 bytes, or bf16 for the unquantized cache -- contiguous.
int check_cache(const pa_tensor* t, const char* name, int64_t* nb, int64_t* hkv) {
  int rc = check_tensor(t, name);
  if (rc) return rc;
  if (t->dtype != PA_DTYPE_U8 && t->dtype != PA_DTYPE_F8E4M3 && t->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, std::string(name) + " must be uint8, float8_e4m3fn or bfloat16");
  if (t->ndim < 3) return fail(PA_ERR_SHAPE, std::string(name) + " must be [num_blocks, Hkv, 16384]");
  int64_t inner = 1;
  for (int i = 2; i < t->ndim; ++i) inner *= t->shape[i];
  if (inner != kBlockBytes)
    return fail(PA_ERR_SHAPE, std::string(name) + ": each (page, head) block must hold 16384 elements (128-token pages, head_dim 128)");
  if (!contiguous(t)) return fail(PA_ERR_LAYOUT, std::string(name) + " must be contiguous");
  if (!aligned(t->data, 16)) return fail(PA_ERR_LAYOUT, std::string(name) + " must be 16-byte aligned");
  *nb = t->shape[0];
  *hkv = t->shape[1];
  return PA_OK;
}

int check_scales(const pa_tensor* ks, const pa_tensor* vs, int mode, int64_t nb, int64_t hkv) {
  if (mode == PA_SCALE_NONE) return PA_OK;
  const pa_tensor* ts[2] = {ks, vs};
  const char* names[2] = {"k_scale", "v_scale"};
  for (int i = 0; i < 2; ++i) {
    int rc = check_tensor(ts[i], names[i]);
    if (rc) return rc;
    if (ts[i]->dtype != PA_DTYPE_F32) return fail(PA_ERR_DTYPE, std::string(names[i]) + " must be float32");
    if (mode == PA_SCALE_SCALAR) {
      if (numel(ts[i]) != 1) return fail(PA_ERR_SHAPE, std::string(names[i]) + " must hold one value in scalar mode");
    } else {
      if (ts[i]->ndim != 3 || ts[i]->shape[0] != nb || ts[i]->shape[1] != hkv || ts[i]->shape[2] != kPage)
        return fail(PA_ERR_SHAPE, std::string(names[i]) + " must be [num_blocks, Hkv, 128] in per-token mode");
      if (!contiguous(ts[i])) return fail(PA_ERR_LAYOUT, std::string(names[i]) + " must be contiguous");
      if (!aligned(ts[i]->data, 16)) return fail(PA_ERR_LAYOUT, std::string(names[i]) + " must be 16-byte aligned");
    }
  }
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Scratch arenas, one per (device, stream).
// Layout: [arrival counters, counter_bytes][split-K partials].  The counter
// region has a fixed size per arena, so partials of one call never land
// where a later call keeps counters; counters are zeroed on allocation and
// every in-kernel merge puts its counters back to zero.
struct Arena {
  void* ptr = nullptr;
  size_t bytes = 0;          // total
  size_t counter_bytes = 0;  // leading counter region
};
std::mutex g_mu;
std::map<std::pair<int, void*>, Arena> g_arenas;
// Arenas replaced by a larger one.  A graph captured while one of them was
// current still holds its address in its kernel arguments, so they stay
// allocated until pa_release.  Each growth at least doubles the arena, so
// the retired ones of a (device, stream) add up to less than the current.
std::vector<std::pair<int, void*>> g_retired;

int get_scratch(hipStream_t stream, size_t need_counters, size_t need_partials, uint32_t** counters,
                void** partials) {
  *counters = nullptr;
  *partials = nullptr;
  if (need_counters == 0 && need_partials == 0) return PA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_mu);
  Arena& ar = g_arenas[{dev, reinterpret_cast<void*>(stream)}];
  if (ar.ptr && ar.counter_bytes >= need_counters && ar.bytes - ar.counter_bytes >= need_partials) {
    *counters = static_cast<uint32_t*>(ar.ptr);
    *partials = static_cast<char*>(ar.ptr) + ar.counter_bytes;
    return PA_OK;
  }
  const size_t cnt = std::max(ar.counter_bytes, need_counters);
  const size_t need = cnt + std::max(ar.ptr ? ar.bytes - ar.counter_bytes : size_t(0), need_partials);
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return fail(PA_ERR_HIP, "hipStreamIsCapturing failed");
  if (st != hipStreamCaptureStatusNone)
    return fail(PA_ERR_NOT_RESERVED,
                "split-K scratch must grow to " + std::to_string(need) +
                    " bytes while the stream is being captured; call pa_reserve before capture");
  size_t sz = 1;
  while (sz < need) sz <<= 1;
  void* fresh = nullptr;
  if (hipMalloc(&fresh, sz) != hipSuccess)
    return fail(PA_ERR_HIP, "hipMalloc of " + std::to_string(sz) + " bytes of split-K scratch failed");
  // counters must start at zero (never reached under capture: growth is refused there)
  if (hipMemsetAsync(fresh, 0, cnt, stream) != hipSuccess) {
    (void)hipFree(fresh);
    return fail(PA_ERR_HIP, "clearing the split-K counters failed");
  }
  // The old arena is retired, not freed: work queued on the stream and any
  // graph captured with it may still use it (see g_retired).
  if (ar.ptr) g_retired.emplace_back(dev, ar.ptr);
  ar.ptr = fresh;
  ar.bytes = sz;
  ar.counter_bytes = cnt;
  *counters = static_cast<uint32_t*>(ar.ptr);
  *partials = static_cast<char*>(ar.ptr) + cnt;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Fixed split-K scratch of pa_decode_noalloc (see `scratch` below): its
// device address on each device, looked up once per device with that
// device current.  In host code the array's name only stands for the
// symbol; kernels must be given this address.
int fixed_scratch(void** out);

// ---------------------------------------------------------------------------
int decode_impl(const pa_tensor* q, const pa_tensor* kc, const pa_tensor* vc, const pa_tensor* ks,
                const pa_tensor* vs, const pa_tensor* bt, const pa_tensor* ctx, const pa_tensor* cu,
                const pa_tensor* sp, int mode, const pa_tensor* out, const pa_decode_opts* opts,
                void* stream_ptr, int32_t* check_report = nullptr, bool no_alloc = false,
                const WriteArgs* fuse = nullptr) {
  if (!fuse) g_err.clear();
  int rc;
  if ((rc = check_tensor(q, "q"))) return rc;
  if (q->dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "q must be bfloat16");
  if (q->ndim != 3) return fail(PA_ERR_SHAPE, "q must be [rows, 16*Hkv, 128]");
  const int64_t rows = q->shape[0], Hq = q->shape[1];
  if (q->shape[2] != kDim) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (Hq % kGroup != 0) return fail(PA_ERR_UNSUPPORTED, "query heads must be 16 per KV head");
  if (q->stride[2] != 1 || q->stride[0] % 8 || q->stride[1] % 8 || !aligned(q->data, 16))
    return fail(PA_ERR_LAYOUT, "q: last dim contiguous, row/head strides multiples of 8, 16-byte aligned");

  int64_t nb = 0, hkv = 0, nb2 = 0, hkv2 = 0;
  if ((rc = check_cache(kc, "k_cache", &nb, &hkv))) return rc;
  if ((rc = check_cache(vc, "v_cache", &nb2, &hkv2))) return rc;
  if (nb2 != nb || hkv2 != hkv) return fail(PA_ERR_SHAPE, "k_cache and v_cache shapes differ");
  if (kc->dtype != vc->dtype) return fail(PA_ERR_DTYPE, "k_cache and v_cache dtypes differ");
  if (nb < 1) return fail(PA_ERR_SHAPE, "the KV cache must hold at least one page");
  if (hkv * kGroup != Hq)
    return fail(PA_ERR_UNSUPPORTED, "q has " + std::to_string(Hq) + " heads but the cache has " +
                                        std::to_string(hkv) + " KV heads: the group must be 16");
  if (mode < PA_SCALE_NONE || mode > PA_SCALE_PER_TOKEN) return fail(PA_ERR_INVALID_ARG, "unknown scale_mode");
  const bool bf16kv = kc->dtype == PA_DTYPE_BF16;
  if (bf16kv && mode != PA_SCALE_NONE)
    return fail(PA_ERR_UNSUPPORTED, "a bfloat16 cache is unquantized: scale_mode must be PA_SCALE_NONE");
  if ((rc = check_scales(ks, vs, mode, nb, hkv))) return rc;

  if ((rc = check_tensor(bt, "block_table"))) return rc;
  if (bt->dtype != PA_DTYPE_I32 || bt->ndim != 2) return fail(PA_ERR_DTYPE, "block_table must be int32 [batch, W]");
  if (bt->stride[1] != 1) return fail(PA_ERR_LAYOUT, "block_table rows must be contiguous");
  const int64_t B = bt->shape[0], W = bt->shape[1];
  if ((rc = check_tensor(ctx, "context_lens"))) return rc;
  if (ctx->dtype != PA_DTYPE_I32 || ctx->ndim != 1 || ctx->shape[0] != B || (B > 1 && ctx->stride[0] != 1))
    return fail(PA_ERR_SHAPE, "context_lens must be contiguous int32 [batch]");
  const bool ragged = cu != nullptr && cu->data != nullptr;
  if (ragged) {
    if ((rc = check_tensor(cu, "cu_seqlens_q"))) return rc;
    if (cu->dtype != PA_DTYPE_I32 || cu->ndim != 1 || cu->shape[0] != B + 1 || cu->stride[0] != 1)
      return fail(PA_ERR_SHAPE, "cu_seqlens_q must be contiguous int32 [batch + 1]");
  }
  int64_t topk = 0;
  const bool sparse = sp != nullptr && sp->data != nullptr;
  if (sparse) {
    if ((rc = check_tensor(sp, "sparse_page_idx"))) return rc;
    if (sp->dtype != PA_DTYPE_I32 || sp->ndim != 2 || sp->shape[0] != rows || sp->stride[1] != 1)
      return fail(PA_ERR_SHAPE, "sparse_page_idx must be int32 [rows, topk] with contiguous rows");
    topk = sp->shape[1];
    if (topk < 1) return fail(PA_ERR_SHAPE, "sparse_page_idx needs topk >= 1");
  }
  if ((rc = check_tensor(out, "out"))) return rc;
  if (out->dtype != PA_DTYPE_BF16 || out->ndim != 3 || out->shape[0] != rows || out->shape[1] != Hq ||
      out->shape[2] != kDim)
    return fail(PA_ERR_SHAPE, "out must be bfloat16 with the shape of q");
  if (out->stride[2] != 1 || out->stride[0] % 8 || out->stride[1] % 8 || !aligned(out->data, 16))
    return fail(PA_ERR_LAYOUT, "out: last dim contiguous, row/head strides multiples of 8, 16-byte aligned");

  pa_config cfg{};
  cfg.num_kv_heads = int32_t(hkv);
  cfg.group_size = kGroup;
  cfg.head_dim = kDim;
  cfg.page_size = kPage;
  cfg.kv_dtype = kc->dtype;
  cfg.scale_mode = mode;
  cfg.rows = rows;
  cfg.batch = B;
  cfg.max_pages = W;
  cfg.topk = topk;
  cfg.ragged = ragged ? 1 : 0;
  cfg.max_q_len = opts ? opts->max_q_len : 0;
  cfg.force_parts = opts ? opts->force_parts : 0;
  cfg.merge_mode = opts ? opts->merge_mode : 0;
  cfg.partition_mode = opts ? opts->partition_mode : 0;
  if (opts && (opts->prefetch_depth < 0 || opts->prefetch_depth > 4))
    return fail(PA_ERR_INVALID_ARG, "prefetch_depth must be in [0, 4]");
  if (opts && opts->workgroup_waves != 0 && opts->workgroup_waves != 4 && opts->workgroup_waves != 8)
    return fail(PA_ERR_INVALID_ARG, "workgroup_waves must be 0, 4 or 8");
  Plan plan;
  std::string perr;
  if ((rc = make_plan(cfg, &plan, &perr))) return fail(rc, perr);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  // pa_decode_write: the new tokens are the query rows.  Calls with short
  // requests write them inside the decode launch (block-sparse ones when
  // every request is a single row); the rest run the writer first.
  bool fused = false;
  if (fuse) {
    if (fuse->tokens != rows)
      return fail(PA_ERR_SHAPE, "k_new holds " + std::to_string(fuse->tokens) + " tokens but q holds " +
                                    std::to_string(rows) + " rows: the new tokens are the query rows");
    if (fuse->hkv != hkv) return fail(PA_ERR_SHAPE, "k_new and the cache differ in KV heads");
    const int64_t lmax = ragged ? (opts ? opts->max_q_len : 0) : (B > 0 ? rows / B : 0);
    // (the fused kernels take the two-page ring; a forced deeper ring runs unfused)
    fused = lmax >= 1 && lmax <= PA_FUSED_WRITE_MAX_Q_LEN && (!sparse || lmax == 1) &&
            !(opts && opts->prefetch_depth > 2);
  }
  if (check_report) {
    // the device-side input check: the same host validation, then the check
    // kernel instead of the decode (no scratch, nothing written but the report)
    if (!aligned(check_report, 4)) return fail(PA_ERR_LAYOUT, "report must be 4-byte aligned");
    DecodeArgs c{};
    c.k_scale = mode == PA_SCALE_NONE ? nullptr : static_cast<const float*>(ks->data);
    c.v_scale = mode == PA_SCALE_NONE ? nullptr : static_cast<const float*>(vs->data);
    c.block_table = static_cast<const int32_t*>(bt->data);
    c.bt_stride = bt->stride[0];
    c.context_lens = static_cast<const int32_t*>(ctx->data);
    c.cu_seqlens_q = ragged ? static_cast<const int32_t*>(cu->data) : nullptr;
    c.sparse_idx = sparse ? static_cast<const int32_t*>(sp->data) : nullptr;
    c.sp_stride = sparse ? sp->stride[0] : 0;
    c.num_blocks = nb;
    c.hkv = int32_t(hkv);
    c.rows = int32_t(rows);
    c.batch = int32_t(B);
    c.width = int32_t(W);
    c.topk = int32_t(topk);
    c.uniform_q_len = ragged ? 0 : int32_t(rows / B);
    c.scale_mode = mode;
    c.kv_bf16 = bf16kv ? 1 : 0;
    hipError_t he = launch_check(c, check_report, stream);
    if (he != hipSuccess) return fail(PA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(he));
    return PA_OK;
  }
  if (rows == 0) return PA_OK;

  uint32_t* counters = nullptr;
  void* partials = nullptr;
  if (no_alloc) {
    // the library's fixed array instead of an arena: never allocates
    if (plan.fused_merge)
      return fail(PA_ERR_UNSUPPORTED,
                  "pa_decode_noalloc: the in-kernel merge needs per-unit counters; use the separate merge kernel");
    const int64_t need = plan.merge ? plan.scratch_bytes - plan.counter_bytes : 0;
    if (need > int64_t(PA_NOALLOC_MAX_SCRATCH_BYTES))
      return fail(PA_ERR_CAPACITY, "pa_decode_noalloc: this call's split-K scratch bucket needs " +
                                       std::to_string(need) + " bytes, above the fixed " +
                                       std::to_string(int64_t(PA_NOALLOC_MAX_SCRATCH_BYTES)) +
                                       "; use pa_decode with pa_reserve");
    if (need > 0 && (rc = fixed_scratch(&partials))) return rc;
  } else if ((rc = get_scratch(stream, size_t(plan.counter_bytes),
                               size_t(plan.scratch_bytes - plan.counter_bytes), &counters, &partials))) {
    return rc;
  }

  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_row_stride = q->stride[0];
  a.q_head_stride = q->stride[1];
  a.k_cache = static_cast<const uint8_t*>(kc->data);
  a.v_cache = static_cast<const uint8_t*>(vc->data);
  a.k_scale = mode == PA_SCALE_NONE ? nullptr : static_cast<const float*>(ks->data);
  a.v_scale = mode == PA_SCALE_NONE ? nullptr : static_cast<const float*>(vs->data);
  a.block_table = static_cast<const int32_t*>(bt->data);
  a.bt_stride = bt->stride[0];
  a.context_lens = static_cast<const int32_t*>(ctx->data);
  a.cu_seqlens_q = ragged ? static_cast<const int32_t*>(cu->data) : nullptr;
  a.sparse_idx = sparse ? static_cast<const int32_t*>(sp->data) : nullptr;
  a.sp_stride = sparse ? sp->stride[0] : 0;
  a.out = static_cast<uint16_t*>(out->data);
  a.out_row_stride = out->stride[0];
  a.out_head_stride = out->stride[1];
  if (plan.merge) {
    const int64_t pairs = plan.balanced ? int64_t(plan.nslot) * plan.lrows * Hq
                                        : int64_t(plan.parts_launched) * rows * Hq;
    a.part_ml = static_cast<float*>(partials);
    a.part_acc = static_cast<float*>(partials) + 2 * pairs;
    a.unit_count = plan.fused_merge ? counters : nullptr;
  }
  a.num_blocks = nb;
  a.hkv = int32_t(hkv);
  a.rows = int32_t(rows);
  a.batch = int32_t(B);
  a.width = int32_t(W);
  a.topk = int32_t(topk);
  a.uniform_q_len = ragged ? 0 : int32_t(rows / B);
  a.rt = plan.rt;
  a.groups = plan.groups;
  a.parts = plan.parts_launched;
  a.ppp = plan.ppp;
  a.scale_mode = mode;
  a.kv_bf16 = bf16kv ? 1 : 0;
  a.xcd_grouped = plan.xcd_grouped ? 1 : 0;
  a.nq = int32_t(plan.nq);
  a.balanced = plan.balanced ? 1 : 0;
  a.nslot = plan.nslot;
  a.lrows = plan.lrows;
  a.prefill = plan.prefill ? 1 : 0;
  a.kv_once = plan.kv_once ? 1 : 0;
  float sm = (opts && opts->sm_scale != 0.0f) ? opts->sm_scale : 1.0f / std::sqrt(float(kDim));
  a.sm_log2 = sm * 1.4426950408889634f;
  if (fused) {
    a.fused = 1;
    a.kn_bf16 = fuse->in_bf16;
    a.k_new = fuse->k_new;
    a.v_new = fuse->v_new;
    a.kn_tok_stride = fuse->k_tok_stride;
    a.kn_head_stride = fuse->k_head_stride;
    a.vn_tok_stride = fuse->v_tok_stride;
    a.vn_head_stride = fuse->v_head_stride;
    a.slots = fuse->slots;
    a.k_cache_w = fuse->k_cache;
    a.v_cache_w = fuse->v_cache;
    a.k_scale_w = fuse->k_scale;
    a.v_scale_w = fuse->v_scale;
  }

  hipEvent_t e0 = opts ? reinterpret_cast<hipEvent_t>(opts->main_begin_event) : nullptr;
  hipEvent_t e1 = opts ? reinterpret_cast<hipEvent_t>(opts->main_end_event) : nullptr;
  const int depth = (opts && opts->prefetch_depth > 0) ? opts->prefetch_depth : plan.depth;
  const int waves = (opts && opts->workgroup_waves > 0) ? opts->workgroup_waves : plan.waves;
  if (fuse && !fused) {
    hipError_t he = launch_write(*fuse, stream);
    if (he != hipSuccess) return fail(PA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(he));
  }
  hipError_t he = launch_decode(a, plan.grid, plan.merge, plan.sparse, depth, waves, e0, e1, stream);
  if (he != hipSuccess) return fail(PA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(he));
  return PA_OK;
}

// Checks the fused writer's norm and rotary arguments (and the query pair)
// and fills the kernel's block.  Every condition is checked before launch.
int check_norm_rope(const pa_norm_rope* nr, const pa_tensor* q, pa_tensor* q_out, int64_t T, int64_t hkv,
                    NormRopeArgs* out) {
  NormRopeArgs n{};
  n.on = 1;
  int rc;
  if ((rc = check_tensor(nr->positions, "positions"))) return rc;
  if (nr->positions->dtype != PA_DTYPE_I64 || nr->positions->ndim != 1 || nr->positions->shape[0] != T ||
      (T > 1 && nr->positions->stride[0] != 1))
    return fail(PA_ERR_SHAPE, "positions must be contiguous int64 [T]");
  n.positions = static_cast<const int64_t*>(nr->positions->data);
  if (nr->rotary_dim < 0 || nr->rotary_dim > kDim || nr->rotary_dim % 4 != 0)
    return fail(PA_ERR_UNSUPPORTED, "rotary_dim must be 0 or a multiple of 4 up to 128");
  n.rot = nr->rotary_dim;
  n.neox = nr->neox ? 1 : 0;
  n.max_pos = 1;
  if (n.rot > 0) {
    const pa_tensor* tabs[2] = {nr->cos, nr->sin};
    const char* names[2] = {"cos", "sin"};
    for (int i = 0; i < 2; ++i) {
      if ((rc = check_tensor(tabs[i], names[i]))) return rc;
      if (tabs[i]->dtype != PA_DTYPE_F32 || tabs[i]->ndim != 2 || tabs[i]->shape[1] != n.rot / 2 ||
          tabs[i]->shape[0] < 1 || tabs[i]->stride[1] != 1)
        return fail(PA_ERR_SHAPE, std::string(names[i]) + " must be float32 [max_pos, rotary_dim/2], rows contiguous");
    }
    if (nr->cos->shape[0] != nr->sin->shape[0]) return fail(PA_ERR_SHAPE, "cos and sin differ in max_pos");
    n.cos = static_cast<const float*>(nr->cos->data);
    n.sin = static_cast<const float*>(nr->sin->data);
    n.cos_stride = nr->cos->stride[0];
    n.sin_stride = nr->sin->stride[0];
    n.max_pos = nr->cos->shape[0];
  }
  const pa_tensor* ws[2] = {nr->k_norm_weight, nr->q_norm_weight};
  const char* wnames[2] = {"k_norm_weight", "q_norm_weight"};
  const float* wp[2] = {nullptr, nullptr};
  for (int i = 0; i < 2; ++i) {
    if (!ws[i] || !ws[i]->data) continue;
    if ((rc = check_tensor(ws[i], wnames[i]))) return rc;
    if (ws[i]->dtype != PA_DTYPE_F32 || numel(ws[i]) != kDim || (ws[i]->ndim == 1 && ws[i]->stride[0] != 1))
      return fail(PA_ERR_SHAPE, std::string(wnames[i]) + " must be contiguous float32 [128]");
    if (!contiguous(ws[i])) return fail(PA_ERR_LAYOUT, std::string(wnames[i]) + " must be contiguous");
    wp[i] = static_cast<const float*>(ws[i]->data);
  }
  n.k_weight = wp[0];
  n.q_weight = wp[1];
  if (!std::isfinite(nr->eps) || nr->eps < 0.0f) return fail(PA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!std::isfinite(nr->weight_offset)) return fail(PA_ERR_INVALID_ARG, "weight_offset must be finite");
  n.eps = nr->eps;
  n.offset = nr->weight_offset;
  const bool has_q = q && q->data;
  const bool has_qo = q_out && q_out->data;
  if (has_q != has_qo) return fail(PA_ERR_INVALID_ARG, "q and q_out are given together or not at all");
  if (has_q) {
    if ((rc = check_tensor(q, "q"))) return rc;
    if ((rc = check_tensor(q_out, "q_out"))) return rc;
    if (q->dtype != PA_DTYPE_F32 && q->dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "q must be float32 or bfloat16");
    if (q_out->dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "q_out must be bfloat16");
    if (q->ndim != 3 || q->shape[0] != T || q->shape[1] != kGroup * hkv || q->shape[2] != kDim)
      return fail(PA_ERR_SHAPE, "q must be [T, 16*Hkv, 128]");
    for (int i = 0; i < 3; ++i)
      if (q_out->ndim != 3 || q_out->shape[i] != q->shape[i]) return fail(PA_ERR_SHAPE, "q_out must have the shape of q");
    const int64_t qes = q->dtype == PA_DTYPE_F32 ? 4 : 2;
    if (q->stride[2] != 1 || q->stride[0] % 2 || q->stride[1] % 2 || !aligned(q->data, uintptr_t(2 * qes)))
      return fail(PA_ERR_LAYOUT, "q: last dim contiguous, even strides, aligned pairs");
    if (q_out->stride[2] != 1 || q_out->stride[0] % 2 || q_out->stride[1] % 2 || !aligned(q_out->data, 4))
      return fail(PA_ERR_LAYOUT, "q_out: last dim contiguous, even strides, 4-byte aligned");
    n.q_in = q->data;
    n.q_tok_stride = q->stride[0];
    n.q_head_stride = q->stride[1];
    n.q_bf16 = q->dtype == PA_DTYPE_BF16 ? 1 : 0;
    n.hq = int32_t(q->shape[1]);
    n.q_out = static_cast<uint16_t*>(q_out->data);
    n.qo_tok_stride = q_out->stride[0];
    n.qo_head_stride = q_out->stride[1];
  }
  *out = n;
  return PA_OK;
}

// Validates a writer call and fills its kernel block (nothing launched).
int prepare_write(const pa_tensor* k_new, const pa_tensor* v_new, const pa_tensor* slot_mapping,
                  pa_tensor* k_cache, pa_tensor* v_cache, pa_tensor* k_scale, pa_tensor* v_scale, int scale_mode,
                  const pa_norm_rope* nr, const pa_tensor* q, pa_tensor* q_out, WriteArgs* out) {
  int rc;

  if ((rc = check_tensor(k_new, "k_new"))) return rc;
  if ((rc = check_tensor(v_new, "v_new"))) return rc;
  if (k_new->dtype != PA_DTYPE_F32 && k_new->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "k_new must be float32 or bfloat16");
  if (v_new->dtype != k_new->dtype) return fail(PA_ERR_DTYPE, "k_new and v_new dtypes differ");
  if (k_new->ndim != 3 || v_new->ndim != 3) return fail(PA_ERR_SHAPE, "k_new, v_new must be [T, Hkv, 128]");
  for (int i = 0; i < 3; ++i)
    if (k_new->shape[i] != v_new->shape[i]) return fail(PA_ERR_SHAPE, "k_new and v_new shapes differ");
  const int64_t T = k_new->shape[0], hkv_in = k_new->shape[1];
  if (k_new->shape[2] != kDim) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
  const int64_t esz = k_new->dtype == PA_DTYPE_F32 ? 4 : 2;
  for (const pa_tensor* t : {k_new, v_new})
    if (t->stride[2] != 1 || t->stride[0] % 2 || t->stride[1] % 2 || !aligned(t->data, uintptr_t(2 * esz)))
      return fail(PA_ERR_LAYOUT, "k_new/v_new: last dim contiguous, even strides, aligned pairs");
  if ((rc = check_tensor(slot_mapping, "slot_mapping"))) return rc;
  if (slot_mapping->dtype != PA_DTYPE_I64 || slot_mapping->ndim != 1 || slot_mapping->shape[0] != T ||
      (T > 1 && slot_mapping->stride[0] != 1))
    return fail(PA_ERR_SHAPE, "slot_mapping must be contiguous int64 [T]");
  int64_t nb = 0, hkv = 0, nb2 = 0, hkv2 = 0;
  if ((rc = check_cache(k_cache, "k_cache", &nb, &hkv))) return rc;
  if ((rc = check_cache(v_cache, "v_cache", &nb2, &hkv2))) return rc;
  if (nb2 != nb || hkv2 != hkv) return fail(PA_ERR_SHAPE, "k_cache and v_cache shapes differ");
  if (hkv != hkv_in) return fail(PA_ERR_SHAPE, "k_new has a different number of KV heads than the cache");
  if (k_cache->dtype != v_cache->dtype) return fail(PA_ERR_DTYPE, "k_cache and v_cache dtypes differ");
  if (scale_mode < PA_SCALE_NONE || scale_mode > PA_SCALE_PER_TOKEN)
    return fail(PA_ERR_INVALID_ARG, "unknown scale_mode");
  const bool bf16kv = k_cache->dtype == PA_DTYPE_BF16;
  if (bf16kv && scale_mode != PA_SCALE_NONE)
    return fail(PA_ERR_UNSUPPORTED, "a bfloat16 cache is unquantized: scale_mode must be PA_SCALE_NONE");
  if ((rc = check_scales(k_scale, v_scale, scale_mode, nb, hkv))) return rc;
  NormRopeArgs nra{};
  if (nr && (rc = check_norm_rope(nr, q, q_out, T, hkv, &nra))) return rc;
  if (T * (hkv + nra.hq) > kMaxGrid) return fail(PA_ERR_CAPACITY, "too many (token, head) pairs for one launch");

  WriteArgs& a = *out;
  a = WriteArgs{};
  a.k_new = k_new->data;
  a.v_new = v_new->data;
  a.k_tok_stride = k_new->stride[0];
  a.k_head_stride = k_new->stride[1];
  a.v_tok_stride = v_new->stride[0];
  a.v_head_stride = v_new->stride[1];
  a.in_bf16 = k_new->dtype == PA_DTYPE_BF16;
  a.out_bf16 = bf16kv ? 1 : 0;
  a.slots = static_cast<const int64_t*>(slot_mapping->data);
  a.k_cache = static_cast<uint8_t*>(k_cache->data);
  a.v_cache = static_cast<uint8_t*>(v_cache->data);
  a.k_scale = scale_mode == PA_SCALE_NONE ? nullptr : static_cast<float*>(k_scale->data);
  a.v_scale = scale_mode == PA_SCALE_NONE ? nullptr : static_cast<float*>(v_scale->data);
  a.num_blocks = nb;
  a.tokens = T;
  a.hkv = int32_t(hkv);
  a.scale_mode = scale_mode;
  a.nr = nra;
  return PA_OK;
}

int write_impl(const pa_tensor* k_new, const pa_tensor* v_new, const pa_tensor* slot_mapping,
               pa_tensor* k_cache, pa_tensor* v_cache, pa_tensor* k_scale, pa_tensor* v_scale, int scale_mode,
               const pa_norm_rope* nr, const pa_tensor* q, pa_tensor* q_out, void* stream) {
  g_err.clear();
  WriteArgs a;
  int rc;
  if ((rc = prepare_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_mode, nr, q, q_out,
                          &a)))
    return rc;
  if (a.tokens == 0) return PA_OK;
  hipError_t he = launch_write(a, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(PA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(he));
  return PA_OK;
}

}  // namespace
}  // namespace fp8pa

// The split-K scratch of pa_decode_noalloc: a fixed array in every device's
// memory, held from the library's load until the process ends.  All calls on
// a device share it (they must not overlap in time), and it keeps the last
// call's contents; nothing in it needs to start at zero, since every partial
// a merge reads is written first by the same call's main kernel.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_MAX_SCRATCH_BYTES];

namespace fp8pa {
namespace {

int fixed_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of `scratch` there
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_HIP, std::string("hipGetSymbolAddress of the fixed scratch failed: ") +
                                  hipGetErrorString(e));
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return PA_OK;
}

}  // namespace
}  // namespace fp8pa

using namespace fp8pa;

extern "C" {

int pa_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
              const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* block_table,
              const pa_tensor* context_lens, const pa_tensor* cu_seqlens_q,
              const pa_tensor* sparse_page_idx, int scale_mode, pa_tensor* out, void* stream) {
  return decode_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, cu_seqlens_q,
                     sparse_page_idx, scale_mode, out, nullptr, stream);
}

int pa_decode_ex(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                 const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* block_table,
                 const pa_tensor* context_lens, const pa_tensor* cu_seqlens_q,
                 const pa_tensor* sparse_page_idx, int scale_mode, pa_tensor* out,
                 const pa_decode_opts* opts, void* stream) {
  return decode_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, cu_seqlens_q,
                     sparse_page_idx, scale_mode, out, opts, stream);
}

int pa_decode_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* block_table,
                      const pa_tensor* context_lens, const pa_tensor* cu_seqlens_q,
                      const pa_tensor* sparse_page_idx, int scale_mode, pa_tensor* out,
                      const pa_decode_opts* opts, void* stream) {
  return decode_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, cu_seqlens_q,
                     sparse_page_idx, scale_mode, out, opts, stream, nullptr, true);
}

int pa_check_decode_inputs(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                           const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* block_table,
                           const pa_tensor* context_lens, const pa_tensor* cu_seqlens_q,
                           const pa_tensor* sparse_page_idx, int scale_mode, const pa_tensor* out,
                           int32_t* report, void* stream) {
  if (!report) return fail(PA_ERR_INVALID_ARG, "report must be a device int32[16] buffer");
  return decode_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, cu_seqlens_q,
                     sparse_page_idx, scale_mode, out, nullptr, stream, report);
}

int pa_decode_write(const pa_tensor* q, const pa_tensor* k_new, const pa_tensor* v_new,
                    const pa_tensor* slot_mapping, pa_tensor* k_cache, pa_tensor* v_cache, pa_tensor* k_scale,
                    pa_tensor* v_scale, const pa_tensor* block_table, const pa_tensor* context_lens,
                    const pa_tensor* cu_seqlens_q, const pa_tensor* sparse_page_idx, int scale_mode,
                    pa_tensor* out, const pa_decode_opts* opts, void* stream) {
  g_err.clear();
  WriteArgs w;
  int rc;
  if ((rc = prepare_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_mode, nullptr,
                          nullptr, nullptr, &w)))
    return rc;
  return decode_impl(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, cu_seqlens_q,
                     sparse_page_idx, scale_mode, out, opts, stream, nullptr, false, &w);
}

int kv_quant_write(const pa_tensor* k_new, const pa_tensor* v_new, const pa_tensor* slot_mapping,
                   pa_tensor* k_cache, pa_tensor* v_cache, pa_tensor* k_scale, pa_tensor* v_scale,
                   int scale_mode, void* stream) {
  return write_impl(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_mode, nullptr,
                    nullptr, nullptr, stream);
}

int kv_norm_rope_write(const pa_tensor* q, pa_tensor* q_out, const pa_tensor* k_new, const pa_tensor* v_new,
                       const pa_tensor* slot_mapping, pa_tensor* k_cache, pa_tensor* v_cache,
                       pa_tensor* k_scale, pa_tensor* v_scale, int scale_mode, const pa_norm_rope* nr,
                       void* stream) {
  if (!nr) return fail(PA_ERR_INVALID_ARG, "kv_norm_rope_write: nr is NULL");
  return write_impl(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_mode, nr, q,
                    q_out, stream);
}
int pa_index_topk(const pa_tensor* q_idx, const pa_tensor* index_cache, const pa_tensor* block_table,
                  const pa_tensor* context_lens, const pa_tensor* cu_seqlens_q, int max_q_len, float sm_scale,
                  pa_tensor* sparse_page_idx, pa_tensor* block_scores, void* stream) {
  g_err.clear();
  int rc;
  if ((rc = check_tensor(q_idx, "q_idx"))) return rc;
  if (q_idx->dtype != PA_DTYPE_BF16) return fail(PA_ERR_DTYPE, "q_idx must be bfloat16");
  if (q_idx->ndim != 2 || q_idx->shape[1] != kDim)
    return fail(PA_ERR_SHAPE, "q_idx must be [rows, 128]");
  const int64_t rows = q_idx->shape[0];
  if (q_idx->stride[1] != 1 || q_idx->stride[0] % 8 || !aligned(q_idx->data, 16))
    return fail(PA_ERR_LAYOUT, "q_idx: last dim contiguous, row stride a multiple of 8, 16-byte aligned");
  if ((rc = check_tensor(index_cache, "index_cache"))) return rc;
  if (index_cache->dtype != PA_DTYPE_U8 && index_cache->dtype != PA_DTYPE_F8E4M3)
    return fail(PA_ERR_DTYPE, "index_cache must be uint8 or float8_e4m3fn");
  if (index_cache->ndim < 2) return fail(PA_ERR_SHAPE, "index_cache must be [num_blocks, 128, 128]");
  int64_t inner = 1;
  for (int i = 1; i < index_cache->ndim; ++i) inner *= index_cache->shape[i];
  if (inner != kBlockBytes) return fail(PA_ERR_SHAPE, "index_cache: each page must hold 128 x 128 bytes");
  if (!contiguous(index_cache) || !aligned(index_cache->data, 16))
    return fail(PA_ERR_LAYOUT, "index_cache must be contiguous and 16-byte aligned");
  const int64_t nb = index_cache->shape[0];
  if (nb < 1) return fail(PA_ERR_SHAPE, "the index cache must hold at least one page");

  if ((rc = check_tensor(block_table, "block_table"))) return rc;
  if (block_table->dtype != PA_DTYPE_I32 || block_table->ndim != 2)
    return fail(PA_ERR_DTYPE, "block_table must be int32 [batch, W]");
  if (block_table->stride[1] != 1) return fail(PA_ERR_LAYOUT, "block_table rows must be contiguous");
  const int64_t B = block_table->shape[0], W = block_table->shape[1];
  if (B < 1 || W < 1) return fail(PA_ERR_SHAPE, "block_table needs batch >= 1 and width >= 1");
  if ((rc = check_tensor(context_lens, "context_lens"))) return rc;
  if (context_lens->dtype != PA_DTYPE_I32 || context_lens->ndim != 1 || context_lens->shape[0] != B ||
      (B > 1 && context_lens->stride[0] != 1))
    return fail(PA_ERR_SHAPE, "context_lens must be contiguous int32 [batch]");
  const bool ragged = cu_seqlens_q != nullptr && cu_seqlens_q->data != nullptr;
  if (ragged) {
    if ((rc = check_tensor(cu_seqlens_q, "cu_seqlens_q"))) return rc;
    if (cu_seqlens_q->dtype != PA_DTYPE_I32 || cu_seqlens_q->ndim != 1 || cu_seqlens_q->shape[0] != B + 1 ||
        cu_seqlens_q->stride[0] != 1)
      return fail(PA_ERR_SHAPE, "cu_seqlens_q must be contiguous int32 [batch + 1]");
  } else if (rows % B != 0) {
    return fail(PA_ERR_SHAPE, "rows " + std::to_string(rows) + " not divisible by batch " + std::to_string(B) +
                                  " and no cu_seqlens_q: a ragged segment needs cu_seqlens_q");
  }
  if (max_q_len < 0) return fail(PA_ERR_INVALID_ARG, "max_q_len must be >= 0");
  if ((rc = check_tensor(sparse_page_idx, "sparse_page_idx"))) return rc;
  if (sparse_page_idx->dtype != PA_DTYPE_I32 || sparse_page_idx->ndim != 2 || sparse_page_idx->shape[0] != rows ||
      sparse_page_idx->stride[1] != 1)
    return fail(PA_ERR_SHAPE, "sparse_page_idx must be int32 [rows, topk] with contiguous rows");
  const int64_t topk = sparse_page_idx->shape[1];
  if (topk < 1) return fail(PA_ERR_SHAPE, "topk must be >= 1");
  if (rows > 1 && sparse_page_idx->stride[0] < topk)
    return fail(PA_ERR_LAYOUT, "sparse_page_idx rows must not overlap");
  if ((rc = check_tensor(block_scores, "block_scores"))) return rc;
  if (block_scores->dtype != PA_DTYPE_F32 || block_scores->ndim != 2 || block_scores->shape[0] != rows ||
      block_scores->shape[1] != W || block_scores->stride[1] != 1)
    return fail(PA_ERR_SHAPE, "block_scores must be float32 [rows, W] with contiguous rows");
  if (rows > 1 && block_scores->stride[0] < W) return fail(PA_ERR_LAYOUT, "block_scores rows must not overlap");
  if (rows > kMaxRows) return fail(PA_ERR_CAPACITY, "rows above " + std::to_string(kMaxRows));
  if (B > kMaxBatch) return fail(PA_ERR_CAPACITY, "batch above " + std::to_string(kMaxBatch));
  if (W > kMaxPages) return fail(PA_ERR_CAPACITY, "block-table width above " + std::to_string(kMaxPages));
  if (topk > kMaxTopk) return fail(PA_ERR_CAPACITY, "topk above " + std::to_string(kMaxTopk));
  int64_t lmax = ragged ? (max_q_len > 0 ? std::min<int64_t>(max_q_len, rows) : rows) : rows / B;
  lmax = std::max<int64_t>(lmax, 1);
  const int64_t groups = (lmax + 15) / 16;
  const int64_t grid = index_score_grid(B * groups, int32_t(W));
  if (grid > int64_t(0x7FFFFFFF))
    return fail(PA_ERR_CAPACITY, "batch x 16-row groups x pages exceeds one launch; give max_q_len");
  if (rows == 0) return PA_OK;

  IndexArgs a{};
  a.q = static_cast<const uint16_t*>(q_idx->data);
  a.q_row_stride = q_idx->stride[0];
  a.index_cache = static_cast<const uint8_t*>(index_cache->data);
  a.num_blocks = nb;
  a.block_table = static_cast<const int32_t*>(block_table->data);
  a.bt_stride = block_table->stride[0];
  a.context_lens = static_cast<const int32_t*>(context_lens->data);
  a.cu_seqlens_q = ragged ? static_cast<const int32_t*>(cu_seqlens_q->data) : nullptr;
  a.scores = static_cast<float*>(block_scores->data);
  a.score_stride = block_scores->stride[0];
  a.out_idx = static_cast<int32_t*>(sparse_page_idx->data);
  a.out_stride = sparse_page_idx->stride[0];
  a.rows = int32_t(rows);
  a.batch = int32_t(B);
  a.width = int32_t(W);
  a.topk = int32_t(topk);
  a.uniform_q_len = ragged ? 0 : int32_t(rows / B);
  a.groups = int32_t(groups);
  const float sm = sm_scale != 0.0f ? sm_scale : 1.0f / std::sqrt(float(kDim));
  a.sm_log2 = sm * 1.4426950408889634f;
  hipError_t he = launch_index(a, grid, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(PA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(he));
  return PA_OK;
}

int pa_query_support(const pa_config* cfg) {
  g_err.clear();
  if (!cfg) return fail(PA_ERR_INVALID_ARG, "cfg is NULL");
  Plan p;
  std::string err;
  int rc = make_plan(*cfg, &p, &err);
  if (rc) return fail(rc, err);
  return PA_OK;
}

int pa_plan_describe(const pa_config* cfg, pa_plan_info* info) {
  g_err.clear();
  if (!cfg || !info) return fail(PA_ERR_INVALID_ARG, "cfg or info is NULL");
  Plan p;
  std::string err;
  int rc = make_plan(*cfg, &p, &err);
  if (rc) return fail(rc, err);
  describe(p, info);
  return PA_OK;
}

int pa_reserve(const pa_config* cfg, void* stream) {
  g_err.clear();
  if (!cfg) return fail(PA_ERR_INVALID_ARG, "cfg is NULL");
  Plan p;
  std::string err;
  int rc = make_plan(*cfg, &p, &err);
  if (rc) return fail(rc, err);
  uint32_t* c = nullptr;
  void* s = nullptr;
  return get_scratch(reinterpret_cast<hipStream_t>(stream), size_t(p.counter_bytes),
                     size_t(p.scratch_bytes - p.counter_bytes), &c, &s);
}

int pa_release(void) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_arenas.empty() && g_retired.empty()) return PA_OK;
  int cur = 0;
  (void)hipGetDevice(&cur);
  int rc = PA_OK;
  std::vector<std::pair<int, void*>> all = g_retired;
  for (auto& kv : g_arenas)
    if (kv.second.ptr) all.emplace_back(kv.first.first, kv.second.ptr);
  for (auto& dp : all) {
    (void)hipSetDevice(dp.first);
    if (hipDeviceSynchronize() != hipSuccess) rc = fail(PA_ERR_HIP, "hipDeviceSynchronize failed");
    (void)hipFree(dp.second);
  }
  g_arenas.clear();
  g_retired.clear();
  (void)hipSetDevice(cur);
  return rc;
}

const char* pa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
