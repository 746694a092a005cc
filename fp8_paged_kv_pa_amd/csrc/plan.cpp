// Configuration checks and the bucketed split-K plan (see plan.h).
#include "plan.h"

#include <algorithm>

namespace fp8pa {

namespace {

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

// Workgroups of a dense grid of `nq` units with `groups` row groups each
// (see the kernel's xcd_group_of): whole rounds of 8 units when there are at
// least 8, so each unit's groups stay on one XCD; otherwise exactly
// nq * groups, spread over the XCDs.
int64_t xcd_grid(int64_t nq, int64_t groups) {
  return nq >= 8 ? ceil_div(nq, 8) * 8 * groups : nq * groups;
}

}  // namespace

int make_plan(const pa_config& c, Plan* out, std::string* err) {
  if (!out) return fail(err, PA_ERR_INVALID_ARG, "plan output is NULL");
  if (c.group_size != kGroup)
    return fail(err, PA_ERR_UNSUPPORTED, "group_size must be 16 query heads per KV head, got " +
                                             std::to_string(c.group_size));
  if (c.head_dim != kDim)
    return fail(err, PA_ERR_UNSUPPORTED, "head_dim must be 128, got " + std::to_string(c.head_dim));
  if (c.page_size != kPage)
    return fail(err, PA_ERR_UNSUPPORTED, "page_size must be 128 tokens, got " +
                                             std::to_string(c.page_size));
  if (c.num_kv_heads < 1 || c.num_kv_heads > kMaxKvHeads)
    return fail(err, PA_ERR_UNSUPPORTED, "num_kv_heads must be in [1, 64], got " +
                                             std::to_string(c.num_kv_heads));
  if (c.kv_dtype != PA_DTYPE_U8 && c.kv_dtype != PA_DTYPE_F8E4M3 && c.kv_dtype != PA_DTYPE_BF16)
    return fail(err, PA_ERR_DTYPE, "KV cache must be uint8 / float8_e4m3fn bytes or bfloat16");
  if (c.scale_mode != PA_SCALE_NONE && c.scale_mode != PA_SCALE_SCALAR &&
      c.scale_mode != PA_SCALE_PER_TOKEN)
    return fail(err, PA_ERR_INVALID_ARG, "unknown scale_mode " + std::to_string(c.scale_mode));
  if (c.kv_dtype == PA_DTYPE_BF16 && c.scale_mode != PA_SCALE_NONE)
    return fail(err, PA_ERR_UNSUPPORTED, "a bfloat16 cache is unquantized: scale_mode must be PA_SCALE_NONE");
  if (c.rows < 0 || c.batch < 1 || c.max_pages < 1 || c.topk < 0)
    return fail(err, PA_ERR_SHAPE, "rows >= 0, batch >= 1, block-table width >= 1, topk >= 0 required");
  if (c.rows > kMaxRows)
    return fail(err, PA_ERR_CAPACITY, "rows " + std::to_string(c.rows) + " above the largest bucket " +
                                          std::to_string(kMaxRows));
  if (c.batch > kMaxBatch)
    return fail(err, PA_ERR_CAPACITY, "batch above " + std::to_string(kMaxBatch));
  if (c.max_pages > kMaxPages)
    return fail(err, PA_ERR_CAPACITY, "block-table width above " + std::to_string(kMaxPages));
  if (c.topk > kMaxTopk)
    return fail(err, PA_ERR_CAPACITY, "topk above " + std::to_string(kMaxTopk));
  if (c.force_parts < 0 || c.force_parts > kMaxParts)
    return fail(err, PA_ERR_INVALID_ARG, "force_parts must be in [0, 256]");
  if (c.max_q_len < 0) return fail(err, PA_ERR_INVALID_ARG, "max_q_len must be >= 0");
  if (c.merge_mode < PA_MERGE_PLAN || c.merge_mode > PA_MERGE_IN_KERNEL)
    return fail(err, PA_ERR_INVALID_ARG, "unknown merge_mode " + std::to_string(c.merge_mode));
  if (c.partition_mode < PA_PARTITION_PLAN || c.partition_mode > PA_PARTITION_BALANCED)
    return fail(err, PA_ERR_INVALID_ARG, "unknown partition_mode " + std::to_string(c.partition_mode));
  // Uniformity is never inferred from divisibility: without cu_seqlens_q the
  // call *declares* every request has rows/batch rows, so rows must divide.
  if (!c.ragged && c.rows % c.batch != 0)
    return fail(err, PA_ERR_SHAPE,
                "rows " + std::to_string(c.rows) + " not divisible by batch " + std::to_string(c.batch) +
                    " and no cu_seqlens_q: a ragged segment needs cu_seqlens_q");

  Plan p;
  p.sparse = c.topk > 0;
  p.bf16kv = c.kv_dtype == PA_DTYPE_BF16;
  const int64_t hkv = c.num_kv_heads;
  int64_t npages;
  if (p.sparse) {
    p.rt = 1;
    p.groups = 1;
    p.lmax = 1;
    p.units = c.rows * hkv;
    npages = c.topk;
  } else {
    int64_t lmax;
    if (!c.ragged) {
      lmax = c.rows / c.batch;
    } else if (c.max_q_len > 0) {
      lmax = std::min<int64_t>(c.max_q_len, c.rows);
    } else {
      lmax = c.rows;  // unknown: the most any one request can own
    }
    lmax = std::max<int64_t>(lmax, 1);
    p.lmax = int(lmax);
    // Long query segments whose length the host knows run the prefill
    // kernel (not with an explicitly requested balanced split or in-kernel
    // merge, which are decode-kernel options).
    const bool lmax_known = !c.ragged || c.max_q_len > 0;
    p.prefill = lmax_known && lmax >= kPrefillMinQ && c.merge_mode != PA_MERGE_IN_KERNEL &&
                c.partition_mode != PA_PARTITION_BALANCED;
    // one or two query rows per workgroup: with two, the accumulators,
    // operands and a two-page prefetch ring fill the 256 VGPRs that let two
    // workgroups share a CU; longer q_len runs as several row groups
    p.rt = p.prefill ? kPrefillPositions : (lmax <= 1 ? 1 : 2);
    p.groups = int(ceil_div(lmax, p.rt));
    // Two-row workgroups read each page once per row group.  With at most
    // two groups the K/V loads are non-temporal, as one-row workgroups' are
    // (measured: q_len 2 and 4, FP8 and bf16, faster steps although the
    // second group's reads then miss the cache more often); with more groups
    // the later groups' cache hits are worth more (q_len 8: slower).
    p.kv_once = !p.prefill && p.rt == 2 && p.groups <= 2;
    p.units = c.batch * hkv * p.groups;
    npages = c.max_pages;
  }

  p.rows_bucket = next_pow2(std::max<int64_t>(c.rows, 1));
  p.pages_bucket = next_pow2(npages);
  p.units_bucket = next_pow2(std::max<int64_t>(p.units, 1));

  int64_t parts;
  if (c.force_parts > 0) {
    parts = c.force_parts;
  } else {
    // (the prefill kernel runs two workgroups per CU)
    parts = std::max<int64_t>(1, (p.prefill ? 2 : 1) * kTargetWorkgroups / p.units_bucket);
  }
  parts = std::min<int64_t>({parts, int64_t(kMaxParts), p.pages_bucket});
  p.parts = int(std::max<int64_t>(parts, 1));
  p.ppp = int(ceil_div(std::max<int64_t>(npages, 1), p.parts));
  p.parts_launched = int(ceil_div(std::max<int64_t>(npages, 1), p.ppp));
  // Two-row workgroups take eight waves (two pages side by side): measured on
  // q_len 4, it streams like twice the partitions without twice the partials.
  // Single-row calls stream best with four.
  p.waves = p.rt == 2 ? 8 : 4;
  p.merge = p.parts_launched > 1;
  p.grid = p.units * p.parts_launched;
  if (!p.sparse && !p.prefill && p.groups > 1) {
    // workgroup id x + 8*(j*groups + gi) carries row group gi of triple
    // 8j + x: the groups of a triple run back to back on one XCD
    p.xcd_grouped = true;
    p.nq = c.batch * hkv * p.parts_launched;
    p.grid = xcd_grid(p.nq, p.groups);
  }
  if (p.merge) {
    // (m, l) pair + 128 accumulators per (partition, row, query head), sized
    // by the bucket so one reservation serves the whole bucket; in front of
    // them one arrival counter per unit for the in-kernel merge.
    const int64_t per = 2 + kDim;
    // The separate merge kernel is the default: measured on MI355X, merging
    // inside the main kernel makes the last partition of each unit a serial
    // tail that pulls every partial through device-coherent loads, which
    // costs more than the extra launch.
    p.fused_merge = c.merge_mode == PA_MERGE_IN_KERNEL;
    p.counter_bytes = (p.units_bucket * 4 + 255) / 256 * 256;
    p.scratch_bytes = p.counter_bytes +
                      int64_t(p.parts) * p.rows_bucket * hkv * kGroup * per * int64_t(sizeof(float));
  }

  // Length-balanced partitions (see pa_partition_mode): nslot slots per (KV
  // head, row group), handed out request by request on the device, each
  // request's partials at (slot, row within the request).  At most
  // nslot - batch slots' worth of pages is spread evenly, so the split
  // always fits.
  const bool can_balance = !p.sparse && !p.prefill && c.batch <= kMaxBalancedBatch && c.force_parts == 0 &&
                           c.merge_mode != PA_MERGE_IN_KERNEL && (!c.ragged || c.max_q_len > 0);
  if (c.partition_mode == PA_PARTITION_BALANCED && !can_balance)
    return fail(err, PA_ERR_UNSUPPORTED,
                "balanced partitions serve dense calls of at most 64 requests (ragged ones with max_q_len), "
                "without force_parts or the in-kernel merge");
  const bool balanced = can_balance && (c.partition_mode == PA_PARTITION_BALANCED ||
                                        (c.partition_mode == PA_PARTITION_PLAN && p.ppp >= kBalanceMinPages));
  if (balanced) {
    const int64_t per_slot = hkv * p.groups;  // workgroups per slot
    p.balanced = true;
    p.nslot = int(std::max<int64_t>(kTargetWorkgroups / per_slot, c.batch + 1));
    p.lrows = p.groups * p.rt;
    p.parts = p.parts_launched = p.nslot;
    p.ppp = 0;
    p.merge = true;
    p.fused_merge = false;
    p.xcd_grouped = p.groups > 1;
    if (p.xcd_grouped) {
      p.nq = int64_t(p.nslot) * hkv;
      p.grid = xcd_grid(p.nq, p.groups);
    } else {
      p.nq = 0;
      p.grid = int64_t(p.nslot) * hkv;
    }
    p.scratch_bytes = p.counter_bytes + next_pow2(p.nslot) * next_pow2(p.lrows) * hkv * kGroup *
                                            int64_t(2 + kDim) * int64_t(sizeof(float));
  }
  if (p.scratch_bytes > kMaxScratchBytes)
    return fail(err, PA_ERR_CAPACITY, "split-K scratch for this bucket exceeds 4 GiB");
  // one launch carries at most 2^31 - 1 workgroups; a ragged call whose
  // max_q_len is unknown plans for rows-long requests and can exceed it
  if (p.grid > kMaxGrid)
    return fail(err, PA_ERR_CAPACITY,
                "the decode grid (" + std::to_string(p.grid) + " workgroups) exceeds one launch" +
                    (c.ragged && c.max_q_len == 0 ? "; give max_q_len for a ragged call" : ""));
  *out = p;
  if (err) err->clear();
  return PA_OK;
}

void describe(const Plan& p, pa_plan_info* info) {
  info->rows_per_group = p.rt;
  info->groups = p.groups;
  info->parts = p.parts_launched;
  info->pages_per_part = p.ppp;
  info->units = p.units;
  info->grid_x = p.grid;
  info->grid_y = 1;
  info->rows_bucket = p.rows_bucket;
  info->pages_bucket = p.pages_bucket;
  info->scratch_bytes = p.scratch_bytes;
  info->merge = p.merge ? 1 : 0;
  info->merge_in_kernel = (p.merge && p.fused_merge) ? 1 : 0;
  info->balanced = p.balanced ? 1 : 0;
}

}  // namespace fp8pa
