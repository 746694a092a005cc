// Kernel argument blocks and launcher entry points shared by the host API
// (api.cpp) and the kernel translation units.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/fp8pa.h"

namespace fp8pa {

// Arguments of the main decode kernel and of the merge kernel.
struct DecodeArgs {
  const uint16_t* q;          // bf16 [rows, Hq, 128]
  int64_t q_row_stride;       // elements
  int64_t q_head_stride;
  const uint8_t* k_cache;     // [num_blocks, Hkv, 16384] FP8 bytes or bf16 elements
  const uint8_t* v_cache;
  const float* k_scale;       // per-token [num_blocks, Hkv, 128] or scalar [1] or null
  const float* v_scale;
  const int32_t* block_table; // [batch, W]
  int64_t bt_stride;
  const int32_t* context_lens;  // [batch]
  const int32_t* cu_seqlens_q;  // [batch+1] or null (uniform)
  const int32_t* sparse_idx;    // [rows, topk] or null
  int64_t sp_stride;
  uint16_t* out;              // bf16 [rows, Hq, 128]
  int64_t out_row_stride;
  int64_t out_head_stride;
  float* part_ml;             // scratch: (m, l) float2 [parts][rows][Hq]; balanced: [nslot][lrows][Hq]
  float* part_acc;            // scratch: float [parts][rows][Hq][128]; balanced: [nslot][lrows][Hq][128]
  uint32_t* unit_count;       // scratch: per-unit arrival counters (in-kernel merge), or null
  int64_t num_blocks;
  int32_t hkv;
  int32_t rows;
  int32_t batch;
  int32_t width;              // block-table width W
  int32_t topk;
  int32_t uniform_q_len;      // rows/batch when cu_seqlens_q is null
  int32_t rt;                 // rows per workgroup (template value, repeated)
  int32_t groups;
  int32_t parts;              // partitions launched per unit
  int32_t ppp;                // pages / list entries per partition
  int32_t scale_mode;
  int32_t kv_bf16;            // 1: unquantized bf16 cache (no scales)
  int32_t xcd_grouped;        // 1: dense grid with a (request, head, partition)'s row groups on one XCD
  int32_t nq;                 // xcd_grouped: (request, KV head, partition) triples, or
                              // (slot, KV head) pairs when balanced
  int32_t balanced;           // 1: length-balanced partitions (slots shared by the requests)
  int32_t nslot;              // balanced: partition slots per (KV head, row group)
  int32_t lrows;              // balanced: rows per request held by a slot's partials
  float sm_log2;              // sm_scale * log2(e)
  // Fused write (pa_decode_write): query row t's own new token k_new[t],
  // v_new[t] sits at position ctx - L + i of its request (i = t - start).
  // The main loop attends only the older positions; the workgroups of the
  // partition holding the request's last position quantize the new tokens
  // with the writer's code, attend them from registers, and (row group 0)
  // store them at slots[t].
  int32_t fused;
  int32_t kn_bf16;            // 1: k_new/v_new are bf16, 0: f32
  const void* k_new;          // [rows, Hkv, 128]
  const void* v_new;
  int64_t kn_tok_stride, kn_head_stride;  // elements
  int64_t vn_tok_stride, vn_head_stride;
  const int64_t* slots;       // [rows]
  uint8_t* k_cache_w;         // the same caches and scales, written
  uint8_t* v_cache_w;
  float* k_scale_w;
  float* v_scale_w;
  // 1: the prefill kernel (long query segments): groups of
  // kPrefillPositions positions, partitions of ppp pages, the fixed split
  int32_t prefill;
  // 1: two-row workgroups load K/V non-temporally (at most two row groups
  // read each page)
  int32_t kv_once;
};

// The key norm and rotary embedding the fused writer applies before the
// cache write (kv_norm_rope_write), and the query it transforms alongside.
struct NormRopeArgs {
  int32_t on;                 // 0: the plain writer
  const int64_t* positions;   // [T]
  const float* cos;           // [max_pos, rot/2] (rows cos_stride apart)
  const float* sin;
  int64_t cos_stride, sin_stride;  // elements
  int64_t max_pos;
  int32_t rot;                // 0 or a multiple of 4 up to 128
  int32_t neox;               // 1: pairs (i, i + rot/2); 0: pairs (2i, 2i + 1)
  const float* k_weight;      // [128] or null (no norm on K)
  const float* q_weight;      // [128] or null
  float eps;
  float offset;               // 0: x_hat * w, 1: x_hat * (1 + w)
  const void* q_in;           // f32 or bf16 [T, Hq, 128], or null
  int64_t q_tok_stride, q_head_stride;
  int32_t q_bf16;
  int32_t hq;
  uint16_t* q_out;            // bf16 [T, Hq, 128]
  int64_t qo_tok_stride, qo_head_stride;
};

struct WriteArgs {
  const void* k_new;          // f32 or bf16 [T, Hkv, 128]
  const void* v_new;
  int64_t k_tok_stride, k_head_stride;  // elements
  int64_t v_tok_stride, v_head_stride;
  int32_t in_bf16;            // 1: inputs are bf16, 0: f32
  int32_t out_bf16;           // 1: the cache is bf16 (stored unquantized)
  const int64_t* slots;       // [T]
  uint8_t* k_cache;           // FP8 bytes, or bf16 elements when out_bf16
  uint8_t* v_cache;
  float* k_scale;             // per-token output, scalar input, or null
  float* v_scale;
  int64_t num_blocks;
  int64_t tokens;
  int32_t hkv;
  int32_t scale_mode;
  NormRopeArgs nr;
};

// Arguments of the sparse-indexer kernels (block scores, then top-k).
struct IndexArgs {
  const uint16_t* q;          // bf16 [rows, 128] index queries
  int64_t q_row_stride;       // elements
  const uint8_t* index_cache; // e4m3fn [num_blocks, 128 tokens, 128 dims], token-major
  int64_t num_blocks;
  const int32_t* block_table; // [batch, W]
  int64_t bt_stride;
  const int32_t* context_lens;  // [batch]
  const int32_t* cu_seqlens_q;  // [batch+1] or null (uniform)
  float* scores;              // f32 [rows, W] (output and work buffer)
  int64_t score_stride;
  int32_t* out_idx;           // int32 [rows, topk]
  int64_t out_stride;
  int32_t rows;
  int32_t batch;
  int32_t width;              // W
  int32_t topk;
  int32_t uniform_q_len;      // rows/batch when cu_seqlens_q is null
  int32_t groups;             // 16-row groups per request
  float sm_log2;              // sm_scale * log2(e)
};

// Launchers (defined with their kernels).  Return hipSuccess or the launch
// error.
hipError_t launch_decode(const DecodeArgs& a, int64_t grid, bool merge, bool sparse, int depth, int waves,
                         hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream);
// The prefill kernel alone (launch_decode calls it for a.prefill, then the merge).
hipError_t launch_prefill_main(const DecodeArgs& a, int64_t grid, hipEvent_t ev_begin, hipEvent_t ev_end,
                               hipStream_t stream);
hipError_t launch_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_index(const IndexArgs& a, int64_t score_grid, hipStream_t stream);
// Workgroups of the block-score kernel for `units` (request, 16-row group) pairs.
int64_t index_score_grid(int64_t units, int32_t width);

}  // namespace fp8pa
