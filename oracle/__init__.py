"""CPU oracle for paged FP8-KV decode attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
anything from this package.  The GPU library never imports, links or calls
it, and it imports nothing from the GPU library: the two share no code,
tables or constants.  Inputs reach both sides from ``workloads`` (seeded
generators that hold none of the method's arithmetic).

What it computes is the plain definition, written out slowly and in fp64:

* ``e4m3``      -- OCP FP8 E4M3 ("fn") decode and round-to-nearest-even,
                   saturating encode, two independent encoders.
* ``layout``    -- the page-shuffled byte order of the K and V pages and the
                   scale arrays, as index functions (page, head, token, dim)
                   -> byte offset.
* ``bf16``      -- bfloat16 decode/encode for the unquantized (BF16) cache.
* ``writer``    -- the cache writer: per (token, KV head) amax/448 scale,
                   fp32 division, e4m3 encode, store through the layout.
* ``attention`` -- softmax attention over the dequantized cache in fp64,
                   for single-row, uniform multi-row, ragged and
                   block-sparse decode, plus the split-K partial/merge form
                   used only to pin the merge identity.
* ``indexer``   -- the sparse indexer that produces the block-sparse page
                   lists: per-page log2-sum-exp block scores over the fp8
                   index cache, and the per-row top-k rule.
* ``norm_rope`` -- the writer fused with the key's RMS norm and rotary
                   embedding: the textbook definitions in fp64, and the
                   fp32 operation order whose output the cache writer takes.

Sources (web pages about serving MiniMax-M3 with an FP8 KV cache on AMD
GPUs):

* ROCm/ATOM pull request 2614 ("general shuffled paged-decode contract"):
  page-shuffled FP8 KV with per-token K/V scales; sections Problem, Change.
* ROCm/ATOM pull request 2710 (FlyDSL paged decode on gfx1250) and its
  review: split-K scratch shapes and capacity buckets ("Must fix" item 1).
* ROCm/ATOM pull request 2122, "fix(minimax-m3): unblock fp8 KV cache and
  EAGLE3 spec decode on the vLLM plugin": section 1 gives the fp8 index
  cache and the block-score product, section 2 the multi-row causal cutoff
  and the ragged-segment rule.
* vllm-project/vllm pull request 52060, "[ROCm][Perf] Fold scalar KV scales
  in MiniMax-M3 sparse attention": section "Suggested Fix" gives the scalar
  scale fold; "Test Plan" compares against a dequantized reference.
* ROCm/ATOM pull request 2710, "Changes" (query/key norm, rotary embedding
  and cache write fused for prefill) and its review, "Smaller" (the
  norm-then-rope and rope-only cache-write branches must share one writer).
"""

from . import bf16, e4m3, layout, writer, attention, indexer, norm_rope  # noqa: F401
