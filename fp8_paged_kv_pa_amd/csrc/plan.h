// Host-side planning for paged decode: configuration checks, the one
// variant-selection table and the capacity-bucketed split-K plan.
//
// Pure C++ (no HIP headers) so it is also built on its own for host-only
// tests.
//
// Bucketing follows ROCm/ATOM pull request 2710's review ("Must fix" 1):
// plans and scratch must come from a bounded set of capacity buckets, not
// one per row count.  Here the partition count and the scratch size depend
// only on power-of-two buckets of (units, pages, rows), so scratch sized
// for a bucket serves every call that falls in it.
#pragma once

#include <cstdint>
#include <string>

#include "../../include/fp8pa.h"

namespace fp8pa {

constexpr int kPage = 128;
constexpr int kDim = 128;
constexpr int kGroup = 16;
constexpr int kBlockBytes = kPage * kDim;

// Capacity limits (largest buckets).  Anything above is refused up front.
constexpr int64_t kMaxRows = 65536;
constexpr int64_t kMaxBatch = 65536;
constexpr int64_t kMaxPages = 1 << 20;   // block-table width (2^27 tokens)
constexpr int64_t kMaxTopk = 4096;
constexpr int32_t kMaxKvHeads = 64;
constexpr int32_t kMaxParts = 256;
constexpr int64_t kMaxScratchBytes = int64_t(4) << 30;
constexpr int64_t kMaxGrid = 0x7FFFFFFF;  // workgroups in one launch

// Workgroups the plan aims for: about one per CU (256 CUs).  Measured on
// the 128K and 8K decode shapes, one long-running 4-wave workgroup per CU
// streams better than several short ones, and fewer partitions mean less
// split-K scratch and a cheaper merge.
constexpr int64_t kTargetWorkgroups = 256;
// Length-balanced partitions: at most one request per lane of a wave, and
// chosen by the plan only where the fixed split gives a workgroup at least
// this many pages (below it the extra memory round trip of the device-side
// split costs more than the balance gains).
constexpr int64_t kMaxBalancedBatch = 64;
constexpr int kBalanceMinPages = 8;

// Long query segments (a prompt run through the decode contract): calls
// whose requests hold at least kPrefillMinQ rows, with that bound known on
// the host (uniform q_len, or max_q_len), run the prefill kernel, whose
// workgroups own kPrefillPositions consecutive positions of one request
// and KV head and share every chunk of K/V among them.  Measured on MI355X
// (4 requests of 4096 tokens): at q_len 32 and 64 the decode kernel's
// balanced split is faster (36.6 / 43.7 us against 48.9 / 56.2), at 128 the
// prefill kernel (66.6 against 89.1 us), and more so for longer prompts.
constexpr int64_t kPrefillMinQ = 128;
constexpr int kPrefillPositions = 8;

struct Plan {
  int rt = 1;              // query positions per workgroup (1 or 2; prefill: kPrefillPositions)
  bool prefill = false;    // the prefill kernel (long query segments)
  int groups = 1;          // row groups per request (dense)
  bool kv_once = false;    // two-row calls of at most two row groups: non-temporal K/V loads
  int parts = 1;           // split-K partitions per unit (scratch is sized for this)
  int parts_launched = 1;  // partitions that can hold work given the real width
  int ppp = 1;             // pages (dense) or list entries (sparse) per partition
  int lmax = 1;            // bound on q_len used by the plan
  int depth = 2;           // pages of KV in flight per wave (chunk-buffer ring)
  int waves = 4;           // waves per workgroup: 4 (one page at a time) or 8 (two side by side)
  bool sparse = false;
  bool bf16kv = false;     // unquantized bf16 cache (32 KiB per page and head)
  bool merge = false;
  bool fused_merge = false; // the last partition of a unit merges (no merge kernel)
  int64_t counter_bytes = 0; // arrival counters at the start of the scratch (fused merge)
  bool xcd_grouped = false;  // dense multi-group grid laid out so row groups share an XCD
  int64_t nq = 0;          // (request, KV head, partition) triples (xcd_grouped)
  int64_t units = 0;       // dense: batch*Hkv*groups; sparse: rows*Hkv
  int64_t grid = 0;        // main-kernel workgroups (1-D)
  int64_t rows_bucket = 1;
  int64_t pages_bucket = 1;
  int64_t units_bucket = 1;
  int64_t scratch_bytes = 0;
  bool balanced = false;   // length-balanced partitions (partition size chosen on the device)
  int nslot = 0;           // balanced: partition slots the requests share
  int lrows = 0;           // balanced: rows per request a slot's partials hold (groups * rt)
};

inline int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks a configuration and builds its plan.  Returns PA_OK or a pa_status
// and fills `err`.
int make_plan(const pa_config& cfg, Plan* plan, std::string* err);

// Fills the public description of a plan.
void describe(const Plan& p, pa_plan_info* info);

}  // namespace fp8pa
