/*
 * fp8pa -- paged-attention decode over a page-shuffled FP8 (OCP e4m3fn) KV
 * cache with per-token K/V scales, for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every argument is a plain pointer or size; tensors travel as
 * `pa_tensor` descriptors (data pointer, dtype, shape, strides in elements).
 * Device tensors live in the memory of the current HIP device.  The caller
 * owns every tensor and the stream; the library keeps no pointer to them
 * after a call returns.  The only memory the library owns is its split-K
 * scratch (see pa_reserve).
 *
 * Sources for the operations (web pages on serving MiniMax-M3 with an FP8
 * KV cache on AMD GPUs):
 *   [ATOM-2614]  ROCm/ATOM pull request 2614 -- general shuffled
 *                paged-decode contract for per-token FP8 KV: sections
 *                "Problem" and "Change".
 *   [ATOM-2710]  ROCm/ATOM pull request 2710 -- FlyDSL paged decode on
 *                gfx1250, and its review ("Must fix" 1: capacity buckets and
 *                split-K scratch; "Should fix" 2: refuse unsupported calls
 *                at startup; "Smaller": one shared cache writer).
 *   [ATOM-2122]  ROCm/ATOM pull request 2122, "fix(minimax-m3): unblock fp8
 *                KV cache and EAGLE3 spec decode on the vLLM plugin",
 *                section 2: multi-row causal cutoff, ragged segments.
 *   [vLLM-52060] vllm-project/vllm pull request 52060, "[ROCm][Perf] Fold
 *                scalar KV scales in MiniMax-M3 sparse attention", section
 *                "Suggested Fix": the scalar-scale fold.
 *
 * ---------------------------------------------------------------------------
 * Fixed geometry: 128-token pages, head dim 128, 16 query heads per KV head
 * (GQA group).  Query head 16*h + j reads KV head h.
 *
 * Cache layout (this library's definition of "page-shuffled"; [ATOM-2614]
 * names the shuffled page without giving its byte order):
 *   k_cache, v_cache: uint8 (or float8_e4m3fn) [num_blocks, Hkv, 16384],
 *     contiguous.  Block (p, h) starts at byte (p*Hkv + h)*16384.  Inside a
 *     block, token slot o (0..127) and dim d (0..127) are at
 *       K: c=o/32, tau=(o%32)/16, r=o%16, j=d/32, g=(d%32)/8, u=d%8,
 *          4096*c + 1024*(2*tau + j/2) + 16*(16*g + r) + 8*(j%2) + u
 *       V: c=o/32, tau=(o%32)/16, w=o%16, g=w/4, e=4*tau + w%4,
 *          delta=d/16, r=d%16,
 *          4096*c + 1024*(delta/2) + 16*(16*g + r) + 8*(delta%2) + e
 *     so each 32-token chunk is one contiguous 4 KiB run and every aligned
 *     16-byte piece is one lane's matrix-core operand.
 *   Unquantized control (the BF16 KV cache the FP8 cache is compared
 *   against, [ATOM-2710] "Test Result"): k_cache, v_cache bfloat16
 *     [num_blocks, Hkv, 16384] contiguous, block (p, h) at element
 *     (p*Hkv + h)*16384, element offsets with the same c, tau, r, j, g, u,
 *     w, e, delta as above:
 *       K: 4096*c + 512*(4*tau + j) + 8*(16*g + r) + u
 *       V: 4096*c + 512*delta + 8*(16*g + r) + e
 *     (each 32-token chunk one 8 KiB run, each 16-byte piece one operand).
 *     A bf16 cache has no scales: scale_mode must be PA_SCALE_NONE.
 *   k_scale, v_scale:
 *     PA_SCALE_PER_TOKEN: float32 [num_blocks, Hkv, 128] contiguous, the
 *       scale of (page, KV head, token slot) ([ATOM-2614] "Problem": one
 *       scale per token for K and for V; "Change": cache and scale views are
 *       collapsed per KV head the same way).
 *     PA_SCALE_SCALAR: float32 with one element each ([vLLM-52060]).
 *     PA_SCALE_NONE: ignored (may be NULL).
 *   Dequantized value = e4m3fn(code) * scale.
 *
 * Which tokens a query row sees ([ATOM-2122] section 2): the rows of a
 * request are consecutive; a request with q_len L owns L rows and its
 * context length counts them, so row i (0-based) attends tokens
 * t < context_len - L + i + 1, capped at block_table width * 128.  q_len is
 * cu_seqlens_q[b+1] - cu_seqlens_q[b] when cu_seqlens_q is given (ragged),
 * else rows / batch for every request (uniform; rows % batch != 0 is an
 * error, never a guess).  A row that sees no token outputs 0.
 */
#ifndef FP8PA_H
#define FP8PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_MAX_DIMS 6

/* Element types of a pa_tensor. */
typedef enum pa_dtype {
  PA_DTYPE_U8 = 1,       /* raw FP8 bytes (caches labelled uint8)           */
  PA_DTYPE_F8E4M3 = 2,   /* OCP float8_e4m3fn                               */
  PA_DTYPE_BF16 = 3,
  PA_DTYPE_F32 = 4,
  PA_DTYPE_I32 = 5,
  PA_DTYPE_I64 = 6
} pa_dtype;

/* Scale modes ([vLLM-52060] "Suggested Fix": no-scale, scalar (its
 * KV_SCALE_MODE 1) and per-token/head). */
typedef enum pa_scale_mode {
  PA_SCALE_NONE = 0,
  PA_SCALE_SCALAR = 1,
  PA_SCALE_PER_TOKEN = 2
} pa_scale_mode;

/* Where split-K partials are combined ([ATOM-2710] review "Must fix" 1
 * names the partial scratch; the combination is the same log-sum-exp in
 * either place). */
typedef enum pa_merge_mode {
  PA_MERGE_PLAN = 0,       /* the library's choice: the separate kernel       */
                           /* (measured faster on MI355X: in the main kernel  */
                           /* the merge becomes a serial tail in which one    */
                           /* workgroup per unit pulls every partial through  */
                           /* device-coherent loads)                          */
  PA_MERGE_SEPARATE = 1,   /* a separate merge kernel after the main kernel   */
  PA_MERGE_IN_KERNEL = 2   /* the last partition of each unit to finish      */
                           /* merges all of them inside the main kernel       */
} pa_merge_mode;

/* How a dense call's pages are cut into split-K partitions.  Fixed: every
 * request gets the same partition count and size, set on the host from the
 * block-table width.  Balanced: one partition size for the whole call,
 * chosen on the device from the context lengths, and each request gets as
 * many partitions as its pages need.  Workgroups then stream about the same
 * number of pages whatever the mix of context lengths.  Balanced serves
 * dense calls of at most 64 requests (uniform, or ragged with max_q_len)
 * with the separate merge kernel and no force_parts. */
typedef enum pa_partition_mode {
  PA_PARTITION_PLAN = 0,     /* the library's choice: balanced where it is   */
                             /* served and the fixed split would give a      */
                             /* workgroup 8 or more pages; fixed otherwise   */
  PA_PARTITION_FIXED = 1,
  PA_PARTITION_BALANCED = 2  /* PA_ERR_UNSUPPORTED where it is not served    */
} pa_partition_mode;

/* Return codes.  Every host-checkable problem is reported before anything is
 * launched ([ATOM-2710] review "Should fix" 2; [ATOM-2614] "Change": decline
 * before the low-level launcher aborts).  pa_last_error() has the text. */
typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* NULL where a tensor is required, bad enum    */
  PA_ERR_DTYPE = -2,         /* wrong element type                           */
  PA_ERR_SHAPE = -3,         /* shapes disagree, or rows % batch with no cu  */
  PA_ERR_LAYOUT = -4,        /* strides / alignment the kernels cannot read  */
  PA_ERR_UNSUPPORTED = -5,   /* geometry other than 128/128/16               */
  PA_ERR_CAPACITY = -6,      /* beyond the largest capacity bucket           */
  PA_ERR_NOT_RESERVED = -7,  /* scratch would have to grow during capture    */
  PA_ERR_HIP = -8            /* a HIP runtime call failed                    */
} pa_status;

/* Tensor descriptor.  Strides are in elements.  `data` is a device pointer
 * for every tensor the kernels read or write. */
typedef struct pa_tensor {
  void* data;
  int32_t dtype;                 /* pa_dtype */
  int32_t ndim;
  int64_t shape[PA_MAX_DIMS];
  int64_t stride[PA_MAX_DIMS];
} pa_tensor;

/* Optional knobs of pa_decode_ex.  Zero-initialise, then set what you need. */
typedef struct pa_decode_opts {
  float sm_scale;          /* 0 => 1/sqrt(128)                                */
  int32_t max_q_len;       /* ragged only: caller-measured max rows per       */
                           /* request (0 => unknown, bounded by rows).  Rows  */
                           /* of a request past it are not computed: with    */
                           /* balanced partitions they come out as zeros,    */
                           /* with fixed ones they are left unspecified      */
  int32_t force_parts;     /* 0 => plan chooses; else split-K partitions      */
  void* main_begin_event;  /* hipEvent_t pair recorded by the main kernel's   */
  void* main_end_event;    /* dispatch (its start and end); may be NULL       */
  int32_t prefetch_depth;  /* 0 => plan chooses; else 2..4 pages of KV in     */
                           /* flight per wave (tuning; depths above 2 apply   */
                           /* to dense calls with 4-wave workgroups)          */
  int32_t workgroup_waves; /* 0 => plan chooses; 4 (a workgroup streams one   */
                           /* page at a time) or 8 (two pages side by side;   */
                           /* two-row calls over a bf16 cache always use 4)   */
  int32_t merge_mode;      /* pa_merge_mode                                   */
  int32_t partition_mode;  /* pa_partition_mode                               */
} pa_decode_opts;

/* Host-side description of a decode call, for capability queries, planning
 * and scratch reservation without any device data. */
typedef struct pa_config {
  int32_t num_kv_heads;    /* Hkv                                            */
  int32_t group_size;      /* query heads per KV head: must be 16            */
  int32_t head_dim;        /* must be 128                                    */
  int32_t page_size;       /* must be 128                                    */
  int32_t kv_dtype;        /* PA_DTYPE_U8, PA_DTYPE_F8E4M3, or PA_DTYPE_BF16 */
                           /* (unquantized; scale_mode must be NONE)         */
  int32_t scale_mode;      /* pa_scale_mode                                  */
  int64_t rows;            /* query rows (sum of q_len)                      */
  int64_t batch;           /* requests                                       */
  int64_t max_pages;       /* block_table width                              */
  int64_t topk;            /* sparse list length; 0 => dense                 */
  int32_t ragged;          /* 1 if cu_seqlens_q is given                     */
  int32_t max_q_len;       /* as pa_decode_opts.max_q_len                    */
  int32_t force_parts;     /* as pa_decode_opts.force_parts                  */
  int32_t merge_mode;      /* as pa_decode_opts.merge_mode                   */
  int32_t partition_mode;  /* as pa_decode_opts.partition_mode               */
} pa_config;

/* The launch plan a config maps to (pa_plan_describe). */
typedef struct pa_plan_info {
  int32_t rows_per_group;  /* query positions one workgroup carries: 1 or 2,
                              or 8 for the prefill kernel (requests of at
                              least 128 rows, their length known: uniform
                              q_len or max_q_len)                          */
  int32_t groups;          /* row groups per request (dense) or 1 (sparse)   */
  int32_t parts;           /* split-K partitions per unit                    */
  int32_t pages_per_part;  /* pages (dense) or list entries (sparse) per part*/
  int64_t units;           /* (request|row) x KV head x group                */
  int64_t grid_x, grid_y;  /* main-kernel grid                               */
  int64_t rows_bucket;     /* capacity bucket of rows (power of two)         */
  int64_t pages_bucket;    /* capacity bucket of pages / topk                */
  int64_t scratch_bytes;   /* split-K scratch this bucket needs (0 if none)  */
  int32_t merge;           /* 1 if partials are merged (parts > 1)           */
  int32_t merge_in_kernel; /* 1: merged inside the main kernel; 0: by the    */
                           /* separate merge kernel (when merge is 1)        */
  int32_t balanced;        /* 1: length-balanced partitions; then parts is   */
                           /* the partition slots the requests share and     */
                           /* pages_per_part is 0 (chosen on the device)     */
} pa_plan_info;

/*
 * pa_decode -- paged decode attention ([ATOM-2614] "Change": dense max-q-len-1
 * per-token FP8 decode through the general shuffled contract, the same
 * contract for sparse decode; [ATOM-2122] section 2: uniform and ragged
 * multi-row decode; [vLLM-52060] "Suggested Fix": scale modes).
 *
 *   q             bf16 [rows, 16*Hkv, 128], last dim contiguous, 16-byte
 *                 aligned rows.
 *   k_cache,
 *   v_cache       u8/f8e4m3 (or bf16, unquantized) [num_blocks, Hkv, 16384]
 *                 contiguous (layouts above), both of one dtype,
 *                 num_blocks >= 1.
 *   k_scale,
 *   v_scale       see "scale" above, per scale_mode.
 *   block_table   int32 [batch, W]: physical page of each logical page.  Only
 *                 entries below ceil(limit/128) (dense) or named by the
 *                 sparse list are read.  Entries outside [0, num_blocks)
 *                 contribute no tokens.
 *   context_lens  int32 [batch]: tokens in each request's context, counting
 *                 the request's own query rows.
 *   cu_seqlens_q  int32 [batch+1] (ragged: row starts, cu[0] = 0,
 *                 cu[batch] = rows, non-decreasing) or NULL (uniform).
 *   sparse_page_idx  int32 [rows, topk] logical page numbers each row attends
 *                 (block-sparse; -1 = padding; no duplicates) or NULL (dense).
 *   scale_mode    pa_scale_mode.
 *   out           bf16 [rows, 16*Hkv, 128], last dim contiguous.
 *   stream        hipStream_t (NULL = default stream).
 *
 * Long query segments -- the per-token-as-decode prefill [ATOM-2614]
 * "Change" runs through this contract -- take a kernel of their own when the
 * call's bound on rows per request (its uniform q_len, or
 * pa_decode_opts.max_q_len) is at least 128: 16 query heads x 8 positions
 * per workgroup share each converted chunk of K/V.  Same results to the
 * decode tolerance; pa_plan_describe reports rows_per_group 8 for such
 * calls.
 *
 * Asynchronous on `stream`; no host synchronisation; graph-capturable once
 * the scratch is reserved (pa_reserve).  Returns PA_OK or a pa_status.
 * Device-side preconditions (not checked on the host): cu_seqlens_q
 * monotone with the stated ends, context_len >= q_len, sparse lists free of
 * duplicates, finite scales.  Violations give unspecified output values but
 * no out-of-bounds access; pa_check_decode_inputs reports them.
 */
int pa_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
              const pa_tensor* k_scale, const pa_tensor* v_scale,
              const pa_tensor* block_table, const pa_tensor* context_lens,
              const pa_tensor* cu_seqlens_q, const pa_tensor* sparse_page_idx,
              int scale_mode, pa_tensor* out, void* stream);

/* pa_decode with options (softmax scale, ragged max q_len hint, forced
 * split-K partitions, timing events).  Same kernels as pa_decode. */
int pa_decode_ex(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                 const pa_tensor* k_scale, const pa_tensor* v_scale,
                 const pa_tensor* block_table, const pa_tensor* context_lens,
                 const pa_tensor* cu_seqlens_q, const pa_tensor* sparse_page_idx,
                 int scale_mode, pa_tensor* out, const pa_decode_opts* opts, void* stream);

/* pa_decode_noalloc -- pa_decode_ex for callers that cannot allocate device
 * memory: code under HIP graph capture without a prior pa_reserve, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, checks,
 * kernels and results as pa_decode_ex; the split-K partials go to a fixed
 * array the library holds in each device's memory for the life of the
 * process (PA_NOALLOC_MAX_SCRATCH_BYTES per device), so the call allocates
 * nothing, on the device or through any library.
 *   Limits: a call whose scratch bucket (pa_plan_info.scratch_bytes, less
 *   the in-kernel-merge counters) exceeds PA_NOALLOC_MAX_SCRATCH_BYTES
 *   returns PA_ERR_CAPACITY; merge_mode PA_MERGE_IN_KERNEL returns
 *   PA_ERR_UNSUPPORTED (it needs counters that start at zero).  Both before
 *   any launch.
 *   Sharing: every call on a device uses the same array, which keeps the
 *   last call's contents.  Calls that overlap in time on one device (on two
 *   streams, or replays of graphs holding such calls) race on it and give
 *   wrong results: serialise them.
 *   The first call on each device looks up the array's address (no stream
 *   work); make it outside graph capture. */
#define PA_NOALLOC_MAX_SCRATCH_BYTES (32u << 20)
int pa_decode_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* k_scale, const pa_tensor* v_scale,
                      const pa_tensor* block_table, const pa_tensor* context_lens,
                      const pa_tensor* cu_seqlens_q, const pa_tensor* sparse_page_idx,
                      int scale_mode, pa_tensor* out, const pa_decode_opts* opts, void* stream);

/* Device-side check of a pa_decode call's inputs -- the preconditions the
 * host cannot see without reading device memory.  The pages keep a kernel-side
 * assert as a backstop for malformed decode metadata (ROCm/ATOM pull request
 * 2122, section 2: ragged query rows mis-mapped as uniform ones, and the
 * assert kept beside the fix); here the check is a separate call that
 * reports instead of trapping, so a caller can run it on suspect batches
 * (debug builds, tests, input replay) while pa_decode itself stays unchanged.
 *
 * Arguments: exactly those of pa_decode (the same host validation runs and
 * returns the same pa_status), plus
 *   report   device int32 [16], caller-owned; written on `stream`:
 *              report[0]      number of violating items found (0 = clean)
 *              report[1]      bitmask over pa_check_kind
 *              report[2 + k]  smallest offending index of kind k, or
 *                             INT32_MAX when kind k did not occur
 *            Read it after synchronising `stream`.
 * Nothing is allocated and no output is written; `out` is only validated.
 * Every read stays inside the tensors the descriptors describe, whatever
 * their device values.  Returns PA_OK or a pa_status. */
typedef enum pa_check_kind {
  PA_CHECK_CU_ENDS = 0,     /* cu_seqlens_q[0] != 0 or cu_seqlens_q[batch] != rows (index 0)    */
  PA_CHECK_CU_ORDER = 1,    /* cu_seqlens_q[b+1] < cu_seqlens_q[b] (index b)                    */
  PA_CHECK_CTX_SHORT = 2,   /* context_lens[b] < the request's q_len (index b)                  */
  PA_CHECK_TABLE_ID = 3,    /* an attended page's block-table id outside [0, num_blocks)
                               (index b * W + logical page)                                       */
  PA_CHECK_SPARSE_ID = 4,   /* a list entry neither -1 nor in [0, W) (index row * topk + i)      */
  PA_CHECK_SPARSE_DUP = 5,  /* a page listed twice in one row (index row)                         */
  PA_CHECK_SCALE = 6        /* per-token scale of an attended token not finite or negative
                               (index b * W + logical page); scalar scale not finite or <= 0
                               (index 0)                                                          */
} pa_check_kind;

int pa_check_decode_inputs(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                           const pa_tensor* k_scale, const pa_tensor* v_scale,
                           const pa_tensor* block_table, const pa_tensor* context_lens,
                           const pa_tensor* cu_seqlens_q, const pa_tensor* sparse_page_idx,
                           int scale_mode, const pa_tensor* out, int32_t* report, void* stream);

/*
 * kv_quant_write -- the single cache writer ([ATOM-2710] review "Smaller":
 * one shared writer; [ATOM-2614] "Problem": page-shuffled FP8 plus
 * per-token K/V scales).
 *
 *   k_new, v_new  f32 or bf16 [T, Hkv, 128], last dim contiguous.
 *   slot_mapping  int64 [T]: page*128 + token slot; negative => skip the
 *                 token; a slot past the cache is skipped too.
 *   k_cache, v_cache  as in pa_decode (written at the named slots only).  A
 *                 bf16 cache stores each value rounded to bf16 (nearest,
 *                 ties to even; bf16 inputs unchanged; NaN stays NaN, quiet,
 *                 sign kept) and takes scale_mode NONE only.
 *   k_scale, v_scale  PER_TOKEN: outputs, f32 [num_blocks, Hkv, 128], scale =
 *                 fl32(amax/448) of the token's 128 values (an all-zero row
 *                 stores 0).  SCALAR: inputs, one f32 each, > 0.  NONE: unused.
 *   Codes: y = fl32(x / scale) (IEEE division; x itself when the scale is 0
 *   or in NONE mode), then e4m3fn round-to-nearest-even with saturation to
 *   +-448; NaN gives 0x7F with the input's sign.
 * Slots must be distinct within one call.  Asynchronous on `stream`.
 */
int kv_quant_write(const pa_tensor* k_new, const pa_tensor* v_new,
                   const pa_tensor* slot_mapping, pa_tensor* k_cache, pa_tensor* v_cache,
                   pa_tensor* k_scale, pa_tensor* v_scale, int scale_mode, void* stream);

/*
 * pa_decode_write -- one decode step: kv_quant_write of the step's new
 * tokens followed by pa_decode_ex over the cache they were written to, with
 * the write done inside the decode launch (one launch fewer per step).  The
 * cache write is the writer's own code ([ATOM-2710] review "Smaller": one
 * shared writer), so the bytes and scales stored are exactly those of
 * kv_quant_write; the attention is that of the decode contract over the
 * written cache ([ATOM-2614] "Change"), within the decode's tolerance.
 *
 * Arguments: those of pa_decode_ex, plus k_new, v_new, slot_mapping as in
 * kv_quant_write, with T == rows:
 *   token t is query row t's own token; row i of request b (rows
 *   cu[b] .. cu[b+1]-1, or the uniform split) sits at position
 *   context_lens[b] - L_b + i, and slot_mapping[t] must be the cache slot
 *   of that position through block_table (block_table[b][pos/128]*128 +
 *   pos%128, >= 0).  context_lens counts the new tokens.
 *   k_cache, v_cache, k_scale, v_scale are written (as kv_quant_write) and
 *   read (as pa_decode).
 * Behaviour: dense calls (FP8 with PER_TOKEN, SCALAR or NONE scales, or a
 * bf16 cache) whose requests hold at most PA_FUSED_WRITE_MAX_Q_LEN rows
 * (uniform split, or max_q_len given in opts for a ragged call) run as one
 * decode launch (plus the merge when split): the workgroups of each
 * request's last partition quantize (bf16 cache: round) its new tokens,
 * row group 0 stores them, and every row attends them from registers while
 * the page stream covers the older positions.  Block-sparse calls
 * (sparse_page_idx as in pa_decode) whose requests are single rows run the
 * same way: partition 0 of each row stores its token, and the row attends
 * it only if the token's page is on its list, as the row would after a
 * separate write.  Every other call (longer or unknown q_len, multi-row
 * sparse calls, a forced prefetch depth above 2) runs kv_quant_write and
 * then pa_decode_ex, with the same results.  Errors: everything the two calls
 * check, plus T != rows (PA_ERR_SHAPE), all before any launch.  Slot
 * preconditions that only device memory shows are the caller's: a slot
 * that does not match its position gives a cache and an output that differ
 * from the two separate calls.  Asynchronous on `stream`.
 */
#define PA_FUSED_WRITE_MAX_Q_LEN 16
int pa_decode_write(const pa_tensor* q, const pa_tensor* k_new, const pa_tensor* v_new,
                    const pa_tensor* slot_mapping, pa_tensor* k_cache, pa_tensor* v_cache,
                    pa_tensor* k_scale, pa_tensor* v_scale, const pa_tensor* block_table,
                    const pa_tensor* context_lens, const pa_tensor* cu_seqlens_q,
                    const pa_tensor* sparse_page_idx, int scale_mode, pa_tensor* out,
                    const pa_decode_opts* opts, void* stream);

/*
 * kv_norm_rope_write -- kv_quant_write fused with the key's RMS norm and
 * rotary position embedding, and the same transform of the query in the
 * same launch ([ATOM-2710] "Changes": query/key norm, rotary embedding and
 * cache write fused for prefill; its review, "Smaller": the norm-then-rope
 * path and the rope-only path repeated one cache-write branch and drifted,
 * so both must go through one writer).  K is transformed in registers and
 * then quantized and stored by exactly the code of kv_quant_write; V is
 * written as it comes.  The pages give no norm or rotary parameters, so all
 * are the caller's (pa_norm_rope).
 *
 *   Per (token t, head): with x the 128 values (bf16 inputs widened),
 *     norm (if a weight is given): y_d = x_d / sqrt(mean(x^2) + eps)
 *       * (weight_offset + w_d)  (weight_offset 0: plain RMS norm, 1: the
 *       Gemma form 1 + w);
 *     rotary (rotary_dim > 0): pairs (i, i + rotary_dim/2) when neox, else
 *       (2i, 2i+1), i < rotary_dim/2; with c = cos[pos_t][i], s =
 *       sin[pos_t][i], the pair (a, b) becomes (a*c - b*s, b*c + a*s); dims
 *       from rotary_dim on pass unchanged.
 *   fp32 order, each step one IEEE operation rounded to nearest even, never
 *   fused: sq_d = x_d*x_d; S = balanced binary tree over d in order (sq_0 +
 *   sq_1, sq_2 + sq_3, ..., then adjacent pairs); inv = 1 / sqrt(S/128 +
 *   eps) (correctly rounded divide and square root); y_d = (x_d*inv) *
 *   (weight_offset + w_d); rotary products rounded, then their difference
 *   or sum.
 *
 *   q, q_out   optional (both or neither): q f32 or bf16 [T, 16*Hkv, 128]
 *              (last dim contiguous, even strides), q_out bf16 of the same
 *              shape: the query after its norm (q_norm_weight) and the same
 *              rotary embedding, rounded to bf16 (nearest even).
 *   k_new .. scale_mode, stream   as kv_quant_write.
 *   nr         the transform's parameters (below).
 * Positions outside [0, max_pos) are clamped into it (device values are not
 * checked on the host).  Everything else is checked before launch.
 * Asynchronous; no allocation.  Returns PA_OK or a pa_status.
 */
typedef struct pa_norm_rope {
  const pa_tensor* positions;      /* int64 [T], contiguous                     */
  const pa_tensor* cos;            /* float32 [max_pos, rotary_dim/2], rows    */
  const pa_tensor* sin;            /* contiguous; may be NULL if rotary_dim 0  */
  int32_t rotary_dim;              /* 0 (no rotary) or a multiple of 4 <= 128  */
  int32_t neox;                    /* 1: pairs (i, i + rotary_dim/2);          */
                                   /* 0: pairs (2i, 2i+1)                      */
  const pa_tensor* k_norm_weight;  /* float32 [128] or NULL (no norm on K)     */
  const pa_tensor* q_norm_weight;  /* float32 [128] or NULL (no norm on q)     */
  float eps;                       /* finite, >= 0                             */
  float weight_offset;             /* finite: 0 plain, 1 Gemma (1 + w)         */
} pa_norm_rope;

int kv_norm_rope_write(const pa_tensor* q, pa_tensor* q_out, const pa_tensor* k_new,
                       const pa_tensor* v_new, const pa_tensor* slot_mapping, pa_tensor* k_cache,
                       pa_tensor* v_cache, pa_tensor* k_scale, pa_tensor* v_scale, int scale_mode,
                       const pa_norm_rope* nr, void* stream);

/*
 * pa_index_topk -- the sparse indexer that produces sparse_page_idx for the
 * block-sparse pa_decode ([ATOM-2122] section 1: the index cache is
 * float8_e4m3fn (num_blocks, 128, 128) and the block score is the fp32
 * product of the index query with the fp8 keys times sm_scale*log2(e);
 * section 2: row i of a q_len-L request sees ctx - L + i + 1 tokens).
 *
 *   q_idx         bf16 [rows, 128], one index query per row; last dim
 *                 contiguous, row stride a multiple of 8, 16-byte aligned.
 *   index_cache   u8/f8e4m3 [num_blocks, 128, 128] contiguous, token-major:
 *                 the key of (page p, token slot o) is the 128 bytes at
 *                 (p*128 + o)*128.  No scale (codes are the key values).
 *   block_table, context_lens, cu_seqlens_q, max_q_len
 *                 as in pa_decode / pa_decode_opts (the same row rules;
 *                 max_q_len only sizes the launch of a ragged call).
 *   sm_scale      0 => 1/sqrt(128).
 *   sparse_page_idx  int32 [rows, topk] output, contiguous rows: the row's
 *                 topk highest-scoring logical pages (ties to the lower page)
 *                 in ascending order, padded with -1 when fewer pages have a
 *                 visible token.  1 <= topk <= 4096.
 *   block_scores  float32 [rows, W] output, contiguous rows, caller-owned
 *                 (also the buffer between the two kernels): score of
 *                 logical page n for the row = log2 of the sum over its
 *                 visible tokens of 2^(sm_scale*log2(e)*<q, k_t>); -inf for
 *                 a page with no visible token or an id outside the cache
 *                 (so every entry past the row's last visible page is -inf).
 *   stream        hipStream_t.
 * Two kernels (scores, then top-k), asynchronous, no allocation (capturable).
 * Returns PA_OK or a pa_status; every check happens before launch.
 */
int pa_index_topk(const pa_tensor* q_idx, const pa_tensor* index_cache,
                  const pa_tensor* block_table, const pa_tensor* context_lens,
                  const pa_tensor* cu_seqlens_q, int max_q_len, float sm_scale,
                  pa_tensor* sparse_page_idx, pa_tensor* block_scores, void* stream);

/* pa_query_support -- can this configuration be served?  Call at startup
 * to refuse a configuration before serving it ([ATOM-2710] review "Should
 * fix" 2).  PA_OK or the error pa_decode would return. */
int pa_query_support(const pa_config* cfg);

/* pa_plan_describe -- host-only dry run: the plan and scratch bucket a
 * configuration maps to.  Plans depend only on the capacity buckets, so the
 * set of distinct plans and scratch sizes is bounded ([ATOM-2710] review
 * "Must fix" 1). */
int pa_plan_describe(const pa_config* cfg, pa_plan_info* info);

/* pa_reserve -- allocate, now, the split-K scratch that `cfg` (and every
 * smaller bucket) needs on the current device for calls on `stream`, so
 * later calls (including ones under graph capture) never allocate.  Scratch
 * is per (device, stream): calls on one stream are serialised by the
 * stream; calls on different streams use different scratch.  A call outside
 * capture that needs a larger bucket than the stream's scratch replaces it
 * with a larger one; the replaced scratch is not freed but kept until
 * pa_release, so a graph captured with it can still be replayed (it keeps
 * the scratch it was captured with).  A call under capture that needs more
 * than is reserved returns PA_ERR_NOT_RESERVED and records nothing.  Do not
 * replay two copies of one graph concurrently.  The scratch starts with one
 * arrival counter per unit for the in-kernel merge: zeroed when the scratch
 * is allocated, and put back to zero by every call that uses it. */
int pa_reserve(const pa_config* cfg, void* stream);

/* pa_release -- free all scratch, current and replaced (synchronises each
 * device first).  Graphs captured before pa_release use freed scratch and
 * must not be replayed after it; capture them again. */
int pa_release(void);

/* Text of the last error on the calling thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8PA_H */
