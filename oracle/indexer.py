"""Reference block scores and per-row top-k page selection (the sparse
indexer that produces the block-sparse decode's page lists), in fp64.

Test infrastructure only (see ``oracle/__init__``).

What the pages fix (ROCm/ATOM pull request 2122, "fix(minimax-m3): unblock
fp8 KV cache and EAGLE3 spec decode on the vLLM plugin"):

* section 1 and its Test Result: the index cache is float8_e4m3fn of shape
  (num_blocks, 128, 128) -- one 128-dim index key per token of a 128-token
  page, one byte per element, no scale;
* section 1: the block-score kernel takes the fp32 dot product of the
  (bf16) index query with the fp8 index keys and multiplies it by
  sm_scale * log2(e);
* section 2: the index top-k kernels map a query row to its request and
  give row i of a q_len-L request the causal cutoff ctx - L + i + 1.

Readings where the pages are silent (each listed in the design notes):

* one index query of 128 dims per query row; one page list per row;
* index keys stored token-major: element (page, token slot o, dim d) at
  byte (page * 128 + o) * 128 + d;
* the score of logical page n for a row is the base-2 log-sum-exp of its
  visible tokens' scaled scores, log2 sum_t 2^(s_t) with
  s_t = sm_scale * log2(e) * <q, k_t> -- the page's share of the row's
  softmax mass.  (A positive factor cannot change a max- or sum-based
  ranking; the log2(e) factor only matters because the scores are
  exponentiated in base 2.)  A page with no visible token scores -inf;
* the top-k of a row is its k highest-scoring pages with a finite score,
  ties going to the lower logical page number, listed in ascending logical
  page order and padded with -1;
* like the decode, the block-table width caps the context and a physical
  page id outside the cache contributes no tokens.
"""

import math

import numpy as np

from . import e4m3
from .attention import row_limit, row_request_map

PAGE = 128
DIM = 128
LOG2E = 1.0 / math.log(2.0)


def index_key_offset(page, slot, dim):
    """Byte offset of index key element (page, token slot, dim)."""
    return (np.asarray(page, dtype=np.int64) * PAGE + slot) * DIM + dim


def block_scores_ref(q_idx, index_cache, block_table, context_lens, cu_seqlens_q=None,
                     sm_scale=None, num_blocks=None):
    """fp64 [rows, W] block scores (log2 domain); -inf where a page has no
    visible token.  q_idx: [rows, 128] (bf16 values as float32);
    index_cache: flat uint8 codes, num_blocks * 128 * 128 bytes."""
    q_idx = np.asarray(q_idx, dtype=np.float64)
    rows = q_idx.shape[0]
    bt = np.asarray(block_table, dtype=np.int64)
    B, W = bt.shape
    if num_blocks is None:
        num_blocks = index_cache.size // (PAGE * DIM)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(DIM)
    c = float(sm_scale) * LOG2E
    out = np.full((rows, W), -np.inf)
    if rows == 0:
        return out
    rb, ri, rL = row_request_map(rows, B, cu_seqlens_q)
    dims = np.arange(DIM)
    for r in range(rows):
        b = int(rb[r])
        lim = min(row_limit(context_lens[b], rL[r], ri[r]), W * PAGE)
        if lim <= 0:
            continue
        for n in range((lim + PAGE - 1) // PAGE):
            P = int(bt[b, n])
            if P < 0 or P >= num_blocks:
                continue
            cnt = min(PAGE, lim - n * PAGE)
            codes = index_cache[index_key_offset(P, np.arange(cnt)[:, None], dims[None, :])]
            s = c * (e4m3.decode(codes) @ q_idx[r])
            m = float(s.max())
            out[r, n] = m + math.log2(float(np.sum(np.exp2(s - m))))
    return out


def topk_ref(scores, topk):
    """[rows, topk] int32: each row's k highest finite scores (ties to the
    lower page number), in ascending page order, padded with -1.  Works on
    any float array (fp64 oracle scores or fp32 kernel scores)."""
    scores = np.asarray(scores)
    rows, W = scores.shape
    out = np.full((rows, topk), -1, dtype=np.int32)
    for r in range(rows):
        finite = np.nonzero(scores[r] > -np.inf)[0]
        # stable sort by descending score keeps ties in ascending page order
        order = finite[np.argsort(-scores[r, finite], kind="stable")]
        pick = np.sort(order[:topk])
        out[r, :len(pick)] = pick
    return out


def block_scores_bruteforce(q_idx, index_cache, block_table, context_lens, cu_seqlens_q=None,
                            sm_scale=None):
    """The same scores by plain loops: exactly rounded dot products and sums
    (math.fsum), one token at a time.  For tiny inputs only."""
    rows = len(q_idx)
    B, W = len(block_table), len(block_table[0])
    nb = len(index_cache) // (PAGE * DIM)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(DIM)
    if cu_seqlens_q is None:
        L = rows // B
        starts = [b * L for b in range(B + 1)]
    else:
        starts = [int(x) for x in cu_seqlens_q]
    out = [[-math.inf] * W for _ in range(rows)]
    for b in range(B):
        L = starts[b + 1] - starts[b]
        for i in range(L):
            r = starts[b] + i
            lim = min(int(context_lens[b]) - L + i + 1, W * PAGE)
            for n in range(W):
                toks = [t for t in range(n * PAGE, (n + 1) * PAGE) if t < lim]
                P = int(block_table[b][n])
                if not toks or P < 0 or P >= nb:
                    continue
                ss = []
                for t in toks:
                    o = t % PAGE
                    dot = math.fsum(float(q_idx[r][d]) *
                                    e4m3.decode_byte(int(index_cache[(P * PAGE + o) * DIM + d]))
                                    for d in range(DIM))
                    ss.append(sm_scale * dot / math.log(2.0))
                m = max(ss)
                out[r][n] = m + math.log2(math.fsum(2.0 ** (x - m) for x in ss))
    return np.array(out)
