// Host-only self-test of the planner (csrc/plan.cpp), built with
// -fsanitize=address,undefined by tests/test_host_sanitized.py.  It walks
// configuration space -- including every error path -- and checks the
// invariants the launch code relies on: the grid covers every page exactly
// once per unit, partitions never exceed the scratch they are sized for,
// and scratch depends only on the capacity buckets.
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <set>
#include <string>
#include <vector>

#include "../../fp8_paged_kv_pa_amd/csrc/plan.h"

using namespace fp8pa;

static int failures = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      ++failures;                                         \
      std::fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
    }                                                     \
  } while (0)

static pa_config base() {
  pa_config c{};
  c.num_kv_heads = 1;
  c.group_size = 16;
  c.head_dim = 128;
  c.page_size = 128;
  c.kv_dtype = PA_DTYPE_U8;
  c.scale_mode = PA_SCALE_PER_TOKEN;
  c.rows = 4;
  c.batch = 4;
  c.max_pages = 72;
  return c;
}

// the C ABI's struct layouts (the Python binding mirrors them)
// The dense multi-group grid as the kernel reads it (a restatement written
// here, not shared with the library): with at least 8 units, id x + 8s is
// row group s % groups of unit 8(s / groups) + x; with fewer, id is row
// group id / nq of unit id % nq.
static long long xcd_grid_ref(long long nq, long long groups) {
  return nq >= 8 ? (nq + 7) / 8 * 8 * groups : nq * groups;
}

static void check_xcd_layout(long long nq, long long groups, long long grid) {
  if (grid > (1 << 20)) return;
  std::vector<unsigned char> seen(size_t(nq * groups), 0);
  std::vector<unsigned char> xcd_used(8, 0);
  for (long long bid = 0; bid < grid; ++bid) {
    long long q, gi;
    if (nq >= 8) {
      const long long x = bid & 7, sidx = bid >> 3;
      gi = sidx % groups;
      q = (sidx / groups) * 8 + x;
      if (q >= nq) continue;
      CHECK(bid % 8 == q % 8, "a unit's groups share an XCD");
    } else {
      q = bid % nq;
      gi = bid / nq;
    }
    CHECK(q < nq && gi < groups, "in range");
    seen[size_t(q * groups + gi)]++;
    xcd_used[size_t(bid % 8)] = 1;
  }
  bool once = true;
  for (unsigned char v : seen) once = once && v == 1;
  CHECK(once, "every (unit, group) exactly once");
  int used = 0;
  for (unsigned char v : xcd_used) used += v;
  CHECK(used == (grid >= 8 ? 8 : int(grid)), "work on every XCD the grid can reach (%d)", used);
}

// The prefill grid as the kernel reads it (restated here): id / (batch * hkv
// * parts) counts row groups down from the last, the rest is (request, KV
// head, partition) with the partition fastest.  Every (group, request,
// head, partition) appears once, and the last groups come first.
static void check_prefill_layout(long long batch, long long hkv, long long groups, long long parts, long long grid) {
  CHECK(grid == batch * hkv * groups * parts, "prefill grid %lld", grid);
  if (grid > (1 << 20)) return;
  std::vector<unsigned char> seen(size_t(grid), 0);
  long long prev_gi = groups;
  for (long long bid = 0; bid < grid; ++bid) {
    const long long per = batch * hkv * parts;
    const long long gi = groups - 1 - bid / per;
    long long rem = bid % per;
    const long long part = rem % parts;
    rem /= parts;
    const long long h = rem % hkv, b = rem / hkv;
    CHECK(gi >= 0 && gi < groups && b < batch && h < hkv, "prefill ids in range");
    CHECK(gi <= prev_gi, "heaviest groups first");
    prev_gi = gi;
    const long long idx = ((gi * batch + b) * hkv + h) * parts + part;
    CHECK(!seen[size_t(idx)], "prefill workgroup twice");
    seen[size_t(idx)] = 1;
  }
}

static_assert(sizeof(pa_tensor) == 8 + 4 + 4 + 6 * 8 * 2, "pa_tensor");
static_assert(sizeof(pa_decode_opts) == 48, "pa_decode_opts");
static_assert(sizeof(pa_config) == 6 * 4 + 4 * 8 + 5 * 4 + 4, "pa_config");
static_assert(sizeof(pa_plan_info) == 4 * 4 + 6 * 8 + 3 * 4 + 4, "pa_plan_info");

int main() {
  std::string err;
  Plan p;
  // error paths
  {
    pa_config c = base();
    c.group_size = 8;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED && !err.empty(), "group");
    c = base(); c.head_dim = 64;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "dim");
    c = base(); c.page_size = 16;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "page");
    c = base(); c.kv_dtype = PA_DTYPE_F32;
    CHECK(make_plan(c, &p, &err) == PA_ERR_DTYPE, "dtype");
    c = base(); c.kv_dtype = PA_DTYPE_BF16;  // unquantized cache: scales refused
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "bf16 with scales");
    c.scale_mode = PA_SCALE_NONE;
    CHECK(make_plan(c, &p, &err) == PA_OK && p.bf16kv, "bf16 without scales");
    c = base(); c.scale_mode = 9;
    CHECK(make_plan(c, &p, &err) == PA_ERR_INVALID_ARG, "mode");
    c = base(); c.rows = 121; c.batch = 31;
    CHECK(make_plan(c, &p, &err) == PA_ERR_SHAPE, "121 rows uniform");
    c.ragged = 1;
    CHECK(make_plan(c, &p, &err) == PA_OK, "121 rows ragged");
    c = base(); c.rows = kMaxRows + 1; c.batch = 1;
    CHECK(make_plan(c, &p, &err) == PA_ERR_CAPACITY, "rows cap");
    c = base(); c.rows = 65536; c.batch = 65536; c.ragged = 1; c.num_kv_heads = 64; c.max_pages = 1024;
    CHECK(make_plan(c, &p, &err) == PA_ERR_CAPACITY && err.find("max_q_len") != std::string::npos,
          "grid beyond one launch");
    c.max_q_len = 1;
    CHECK(make_plan(c, &p, &err) == PA_OK && p.grid <= kMaxGrid, "grid with max_q_len");
    c = base(); c.force_parts = 300;
    CHECK(make_plan(c, &p, &err) == PA_ERR_INVALID_ARG, "force parts");
    c = base(); c.batch = 0;
    CHECK(make_plan(c, &p, &err) == PA_ERR_SHAPE, "batch 0");
    CHECK(make_plan(base(), nullptr, &err) == PA_ERR_INVALID_ARG, "null plan");
  }
  // invariants over a grid of configurations
  std::set<long long> scratch_by_bucket[32];
  for (int hkv : {1, 2, 8}) {
    for (long long batch : {1LL, 2LL, 3LL, 4LL, 31LL, 32LL, 33LL, 100LL, 4096LL}) {
      for (int L : {1, 2, 3, 4, 6, 300}) {
        for (long long W : {1LL, 2LL, 5LL, 72LL, 256LL, 1024LL, 3000LL}) {
          for (long long topk : {0LL, 1LL, 32LL, 100LL}) {
            for (int fp : {0, 1, 3, 64}) {
              pa_config c = base();
              c.num_kv_heads = hkv;
              c.batch = batch;
              c.rows = batch * L;
              c.max_pages = W;
              c.topk = topk;
              c.force_parts = fp;
              c.merge_mode = (fp % 3 == 0) ? PA_MERGE_IN_KERNEL : PA_MERGE_PLAN;
              if (c.rows > kMaxRows) continue;
              int rc = make_plan(c, &p, &err);
              if (rc == PA_ERR_CAPACITY && fp > 0) {
                // a forced partition count may ask for more scratch than the
                // largest bucket allows; it must be refused, never truncated
                const long long pb = next_pow2(topk ? topk : W);
                const long long parts = std::min<long long>(std::min<long long>(fp, kMaxParts), pb);
                const bool pf = !topk && L >= kPrefillMinQ && c.merge_mode != PA_MERGE_IN_KERNEL;
                const long long per = pf ? kPrefillPositions : 2;
                const long long units = topk ? c.rows * hkv : batch * hkv * ((L + per - 1) / per);
                const long long counters = (next_pow2(units) * 4 + 255) / 256 * 256;
                const long long want = counters + parts * next_pow2(c.rows) * hkv * 16 * 130 * 4;
                CHECK(want > kMaxScratchBytes, "refused although %lld bytes fit", want);
                continue;
              }
              CHECK(rc == PA_OK, "plan rc %d (%s) fp=%d rows=%lld hkv=%d W=%lld topk=%lld", rc, err.c_str(),
                    fp, (long long)c.rows, hkv, W, topk);
              if (rc) continue;
              const long long npages = topk ? topk : W;
              // long known q_len (uniform here) runs the prefill kernel, except
              // with the in-kernel merge, which only the decode kernel has
              const bool want_pf = !topk && L >= kPrefillMinQ && c.merge_mode != PA_MERGE_IN_KERNEL;
              CHECK(p.prefill == want_pf, "prefill choice L=%d merge=%d", L, c.merge_mode);
              CHECK(p.rt == (topk ? 1 : (want_pf ? kPrefillPositions : (L == 1 ? 1 : 2))), "rt %d", p.rt);
              if (p.prefill) {
                CHECK(!p.xcd_grouped && !p.balanced && p.waves == 4, "prefill layout");
                check_prefill_layout(batch, hkv, p.groups, p.parts_launched, p.grid);
              }
              CHECK(p.groups * p.rt >= (topk ? 1 : L), "groups");
              // non-temporal two-row loads: at most two row groups per page
              CHECK(p.kv_once == (!topk && !want_pf && L >= 2 && L <= 4), "kv_once L=%d", L);
              CHECK(p.parts_launched >= 1 && p.parts_launched <= p.parts, "parts %d/%d", p.parts_launched, p.parts);
              CHECK(p.parts <= kMaxParts, "parts cap");
              // every page position covered once: [k*ppp, (k+1)*ppp) for k < parts_launched
              CHECK((long long)p.ppp * p.parts_launched >= npages, "coverage");
              CHECK((long long)p.ppp * (p.parts_launched - 1) < npages, "no empty tail partition");
              CHECK(p.merge == (p.parts_launched > 1), "merge flag");
              const long long units = topk ? c.rows * hkv : batch * hkv * p.groups;
              CHECK(p.units == units, "units");
              CHECK(p.grid >= 1 && p.grid <= kMaxGrid, "grid within one launch");
              if (!p.xcd_grouped) {
                CHECK(p.grid == units * p.parts_launched, "grid");
              } else {
                // the XCD-grouped layout covers every (triple, row group) once
                CHECK(!topk && p.groups > 1, "xcd layout only for dense multi-group calls");
                CHECK(p.nq == batch * hkv * p.parts_launched, "triples");
                CHECK(p.grid == xcd_grid_ref(p.nq, p.groups), "xcd grid");
                check_xcd_layout(p.nq, p.groups, p.grid);
              }
              if (p.merge) {
                const long long need = (long long)p.parts_launched * c.rows * 16 * hkv * 130 * 4;
                CHECK(p.scratch_bytes - p.counter_bytes >= need, "scratch %lld < %lld",
                      (long long)(p.scratch_bytes - p.counter_bytes), need);
                // one 4-byte arrival counter per unit, 256-byte aligned region
                CHECK(p.counter_bytes >= p.units * 4 && p.counter_bytes % 256 == 0, "counters");
                CHECK(p.fused_merge == (c.merge_mode == PA_MERGE_IN_KERNEL), "merge mode");
              } else {
                CHECK(p.scratch_bytes == 0, "no scratch without merge");
              }
              CHECK(p.rows_bucket >= c.rows && (p.rows_bucket & (p.rows_bucket - 1)) == 0, "rows bucket");
            }
          }
        }
      }
    }
  }
  // scratch depends only on buckets: all row counts in one bucket (lo, 2lo]
  // (the rows that round up to the same power of two) agree
  for (long long lo = 1; lo <= 2048; lo *= 2) {
    std::set<long long> sizes;
    for (long long r = lo + 1; r <= 2 * lo; ++r) {
      pa_config c = base();
      c.rows = r;
      c.batch = r;
      c.max_pages = 1024;
      if (make_plan(c, &p, &err) == PA_OK) sizes.insert(p.scratch_bytes);
    }
    CHECK(sizes.size() == 1, "bucket (%lld, %lld] has %zu scratch sizes", lo, 2 * lo, sizes.size());
  }
  // length-balanced partitions: when the plan chooses them, what it lays out
  for (int hkv : {1, 2, 8}) {
    for (long long batch : {1LL, 3LL, 31LL, 63LL, 64LL, 65LL}) {
      for (int L : {1, 2, 4, 6, 300, 16384}) {
        for (long long W : {1LL, 5LL, 72LL, 256LL, 1024LL, 3000LL}) {
          for (int mode : {PA_PARTITION_PLAN, PA_PARTITION_FIXED, PA_PARTITION_BALANCED}) {
            pa_config c = base();
            c.num_kv_heads = hkv;
            c.batch = batch;
            c.rows = batch * L;
            c.max_pages = W;
            c.partition_mode = mode;
            if (c.rows > kMaxRows) continue;
            Plan fixed;
            pa_config cf = c;
            cf.partition_mode = PA_PARTITION_FIXED;
            CHECK(make_plan(cf, &fixed, &err) == PA_OK && !fixed.balanced, "fixed plan");
            const int rc = make_plan(c, &p, &err);
            if (mode == PA_PARTITION_BALANCED && batch > kMaxBalancedBatch) {
              CHECK(rc == PA_ERR_UNSUPPORTED, "balanced beyond 64 requests refused");
              continue;
            }
            if (rc == PA_ERR_CAPACITY) {
              // a balanced split whose bucketed scratch exceeds the largest bucket
              const long long groups = (L + 1) / 2, rt = L > 1 ? 2 : 1;
              const long long nslot = std::max<long long>(kTargetWorkgroups / (hkv * groups), batch + 1);
              const long long want = next_pow2(nslot) * next_pow2(groups * rt) * hkv * 16 * 130 * 4;
              CHECK(want > kMaxScratchBytes, "balanced refused although %lld bytes fit", want);
              continue;
            }
            CHECK(rc == PA_OK, "balanced plan rc %d (%s)", rc, err.c_str());
            // (an explicitly balanced split keeps the decode kernel; otherwise
            // long q_len runs the prefill kernel, which takes the fixed split)
            CHECK(p.prefill == (mode != PA_PARTITION_BALANCED && L >= kPrefillMinQ), "prefill choice");
            const bool want = batch <= kMaxBalancedBatch && !p.prefill &&
                              (mode == PA_PARTITION_BALANCED ||
                               (mode == PA_PARTITION_PLAN && fixed.ppp >= kBalanceMinPages));
            CHECK(p.balanced == want, "balanced choice batch=%lld W=%lld mode=%d", batch, W, mode);
            if (!p.balanced) continue;
            const long long per_slot = hkv * p.groups;
            CHECK(p.nslot == std::max<long long>(kTargetWorkgroups / per_slot, batch + 1), "slots");
            CHECK(p.nslot > batch, "more slots than requests");
            CHECK(p.lrows == p.groups * p.rt && p.lrows >= L, "rows per slot");
            CHECK(p.merge && !p.fused_merge, "balanced merges in the merge kernel");
            const long long need = (long long)p.nslot * p.lrows * 16 * hkv * 130 * 4;
            CHECK(p.scratch_bytes - p.counter_bytes >= need, "balanced scratch");
            if (p.groups > 1) {
              CHECK(p.xcd_grouped && p.nq == (long long)p.nslot * hkv, "balanced pairs");
              CHECK(p.grid == xcd_grid_ref(p.nq, p.groups), "balanced xcd grid");
              check_xcd_layout(p.nq, p.groups, p.grid);
            } else {
              CHECK(!p.xcd_grouped && p.grid == (long long)p.nslot * hkv, "balanced grid");
            }
          }
        }
      }
    }
  }
  {
    // refusals of a forced balanced split
    pa_config c = base();
    c.partition_mode = PA_PARTITION_BALANCED;
    c.topk = 8;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "balanced sparse");
    c = base(); c.partition_mode = PA_PARTITION_BALANCED; c.force_parts = 4;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "balanced with force_parts");
    c = base(); c.partition_mode = PA_PARTITION_BALANCED; c.merge_mode = PA_MERGE_IN_KERNEL;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "balanced with the in-kernel merge");
    c = base(); c.partition_mode = PA_PARTITION_BALANCED; c.ragged = 1;
    CHECK(make_plan(c, &p, &err) == PA_ERR_UNSUPPORTED, "balanced ragged without max_q_len");
    c.max_q_len = 1;
    CHECK(make_plan(c, &p, &err) == PA_OK && p.balanced, "balanced ragged with max_q_len");
    c = base(); c.partition_mode = 3;
    CHECK(make_plan(c, &p, &err) == PA_ERR_INVALID_ARG, "unknown partition mode");
  }
  {
    // A host model of the device-side split (the bisection for the common
    // partition size): its upper end always fits, the result is the
    // smallest size that fits, and every page lands in exactly one slot.
    unsigned long long rng = 12345;
    auto next = [&]() { rng = rng * 6364136223846793005ULL + 1442695040888963407ULL; return rng >> 33; };
    for (int trial = 0; trial < 4000; ++trial) {
      const int batch = 1 + int(next() % 64);
      const int nslot = std::max(int(1 + next() % 256), batch + 1);
      const int width = 1 + int(next() % 2048);
      std::vector<int> np(batch);
      long long total = 0;
      for (int j = 0; j < batch; ++j) {
        const int kind = int(next() % 4);
        const long long ctx = kind == 0 ? 0 : (long long)(next() % (kind == 1 ? 300 : width * 128 + 500));
        np[j] = int((std::max(0LL, std::min(ctx, (long long)width * 128)) + 127) / 128);
        total += np[j];
      }
      auto count = [&](long long ppp) {
        long long s = 0;
        for (int v : np) s += std::max(1LL, (v + ppp - 1) / ppp);
        return s;
      };
      long long lo = std::max(1LL, (total + nslot - 1) / nslot);
      const long long hi0 = std::max(lo, (total + nslot - batch - 1) / (nslot - batch));
      CHECK(count(hi0) <= nslot, "upper end fits (batch %d, slots %d)", batch, nslot);
      long long hi = hi0;
      while (lo < hi) {
        const long long mid = (lo + hi) / 2;
        if (count(mid) <= nslot) hi = mid; else lo = mid + 1;
      }
      CHECK(count(lo) <= nslot && (lo == 1 || count(lo - 1) > nslot), "smallest fitting size");
      long long covered = 0, slots = 0;
      for (int v : np) {
        const long long parts = std::max(1LL, (v + lo - 1) / lo);
        for (long long k = 0; k < parts; ++k) covered += std::max(0LL, std::min<long long>(lo, v - k * lo));
        slots += parts;
      }
      CHECK(covered == total && slots <= nslot, "pages covered once");
    }
  }
  pa_plan_info info{};
  make_plan(base(), &p, &err);
  describe(p, &info);
  CHECK(info.parts == p.parts_launched && info.grid_x == p.grid && info.merge == (p.merge ? 1 : 0) &&
            info.balanced == (p.balanced ? 1 : 0), "describe");
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("plan self-test ok\n");
  return 0;
}
