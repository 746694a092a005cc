"""Reference paged decode attention over the FP8 cache, in fp64.

Test infrastructure only (see ``oracle/__init__``).

The method (ROCm/ATOM pull request 2614, sections Problem and Change; vLLM
pull request 52060, "Suggested Fix" and "Test Plan") reaches exactly the
plain result: softmax attention over the dequantized cache.  So this module
is that definition written out:

1. decode every attended e4m3 byte exactly (``e4m3.decode``);
2. multiply by its scale: per-token mode the (page, KV head, token) fp32
   scale, scalar mode the one K or V scale, no-scale mode 1;
3. per query row and query head, s_t = sm_scale * <q, k_t> in fp64, then
   out = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s).

Query heads: head ``16*h + j`` (j in 0..15) reads KV head ``h`` (grouped
query attention with 16 query heads per KV head; ROCm/ATOM pull request
2122, section 2, prints the query view [requests, q_len, 1, 16, 128]).

Which tokens a row attends (ROCm/ATOM pull request 2122, section 2): rows
of a request are consecutive; a request with q_len L contributes L rows and
its context length counts those rows, so row i (0-based) of the request sees
tokens t < ctx - L + i + 1.  q_len comes from ``cu_seqlens_q`` when given
(ragged), else every request has rows/B rows (uniform).  The block-sparse
variant attends, for each row, only the logical pages in that row's list
(entries < 0 are padding), with the same per-row cutoff inside each page.

Readings where the pages are silent: a row with no attended token outputs
0; a logical page at or past the block-table width, or a physical page id
outside the cache, contributes no tokens.
"""

import math

import numpy as np

from . import bf16, e4m3, layout

NONE, SCALAR, PER_TOKEN = 0, 1, 2
GROUP = 16
DIM = 128
PAGE = 128


def row_request_map(rows: int, batch: int, cu_seqlens_q=None):
    """For each query row: (request b, index i within the request, q_len L)."""
    if cu_seqlens_q is None:
        if rows % batch != 0:
            raise ValueError("uniform decode needs rows divisible by the batch")
        L = rows // batch
        b = np.arange(rows) // L
        return b, np.arange(rows) % L, np.full(rows, L)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    assert cu.shape == (batch + 1,) and cu[0] == 0 and cu[-1] == rows
    assert np.all(np.diff(cu) >= 0)
    b = np.searchsorted(cu, np.arange(rows), side="right") - 1
    return b, np.arange(rows) - cu[b], (cu[1:] - cu[:-1])[b]


def row_limit(ctx: int, L: int, i: int) -> int:
    """Number of leading tokens row i of a q_len-L request sees."""
    return int(ctx) - int(L) + int(i) + 1


def _dequant_pages(cache_flat, scale_flat, pages, head, Hkv, kind, mode, scalar, kv_dtype="fp8"):
    """Dequantized [len(pages)*128, 128] fp64 rows of the given physical pages.
    kv_dtype "bf16": the cache holds bf16 elements (uint16), no scales."""
    pages = np.asarray(pages, dtype=np.int64)
    if kv_dtype == "bf16":
        idx = (pages * Hkv + head)[:, None, None] * layout.BLOCK_BYTES + (
            layout.K_IDX_BF16 if kind == "k" else layout.V_IDX_BF16)[None]
        return bf16.decode(cache_flat[idx]).reshape(-1, DIM)
    idx = layout.block_base(pages, head, Hkv)[:, None, None] + (
        layout.K_IDX if kind == "k" else layout.V_IDX)[None]
    vals = e4m3.decode(cache_flat[idx]).reshape(-1, DIM)
    if mode == PER_TOKEN:
        sidx = layout.scale_index(pages[:, None], head, np.arange(PAGE)[None, :], Hkv)
        vals = vals * scale_flat[sidx].astype(np.float64).reshape(-1, 1)
    elif mode == SCALAR:
        vals = vals * float(scalar)
    return vals


def _softmax_attend(qv, k, v, sm_scale):
    if k.shape[0] == 0:
        return np.zeros(DIM)
    s = sm_scale * (k @ qv)
    w = np.exp(s - s.max())
    return (w @ v) / w.sum()


def _row_tokens(b, i, L, ctx, block_table, num_blocks, sparse_row):
    """(physical page, first token slot, token count) runs attended by one row."""
    W = block_table.shape[1]
    limit = min(row_limit(ctx[b], L, i), W * PAGE)
    runs = []
    if sparse_row is None:
        pages = range(0, max(0, -(-limit // PAGE)))
    else:
        pages = [int(n) for n in sparse_row if 0 <= int(n) < W]
    for n in pages:
        lo, hi = n * PAGE, min((n + 1) * PAGE, limit)
        if hi <= lo:
            continue
        P = int(block_table[b, n])
        if P < 0 or P >= num_blocks:
            continue
        runs.append((P, n, hi - lo))
    return runs


def attention_ref(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                  cu_seqlens_q=None, sparse_page_idx=None, mode=PER_TOKEN,
                  num_kv_heads=1, sm_scale=None, rows_subset=None, kv_dtype="fp8"):
    """fp64 attention output [rows, 16*Hkv, 128] (or only ``rows_subset``).

    q: [rows, 16*Hkv, 128] values (bf16 inputs widened exactly).
    k_cache, v_cache: flat uint8; k_scale, v_scale: flat float32 (per-token),
    1-element (scalar) or None (no-scale).  block_table int [B, W];
    context_lens int [B]; cu_seqlens_q int [B+1] or None; sparse_page_idx
    int [rows, topk] of logical page numbers or None.
    """
    q = np.asarray(q, dtype=np.float64)
    rows, Hq, D = q.shape
    Hkv = num_kv_heads
    assert Hq == GROUP * Hkv and D == DIM
    block_table = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    B = block_table.shape[0]
    num_blocks = k_cache.size // (Hkv * layout.BLOCK_BYTES)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(DIM)
    if kv_dtype == "bf16":
        mode = NONE
    ks = vs = None
    if mode == SCALAR:
        ks = float(np.asarray(k_scale).reshape(-1)[0])
        vs = float(np.asarray(v_scale).reshape(-1)[0])
    bmap, imap, Lmap = row_request_map(rows, B, cu_seqlens_q)
    sel = np.arange(rows) if rows_subset is None else np.asarray(rows_subset)
    out = np.zeros((len(sel), Hq, DIM))
    cache = {}
    for oi, r in enumerate(sel):
        b, i, L = int(bmap[r]), int(imap[r]), int(Lmap[r])
        sp = None if sparse_page_idx is None else np.asarray(sparse_page_idx)[r]
        runs = _row_tokens(b, i, L, ctx, block_table, num_blocks, sp)
        for h in range(Hkv):
            ks_parts, vs_parts = [], []
            for (P, n, cnt) in runs:
                key = (P, h)
                if key not in cache:
                    cache[key] = (
                        _dequant_pages(k_cache, k_scale, [P], h, Hkv, "k", mode, ks, kv_dtype),
                        _dequant_pages(v_cache, v_scale, [P], h, Hkv, "v", mode, vs, kv_dtype))
                kp, vp = cache[key]
                ks_parts.append(kp[:cnt])
                vs_parts.append(vp[:cnt])
            k = np.concatenate(ks_parts) if ks_parts else np.zeros((0, DIM))
            v = np.concatenate(vs_parts) if vs_parts else np.zeros((0, DIM))
            for j in range(GROUP):
                out[oi, GROUP * h + j] = _softmax_attend(q[r, GROUP * h + j], k, v, sm_scale)
        if len(cache) > 4096:
            cache.clear()
    return out


def attention_ref_scalar_folded(q, k_cache, v_cache, k_scale, v_scale, block_table,
                                context_lens, cu_seqlens_q=None, sparse_page_idx=None,
                                num_kv_heads=1, sm_scale=None):
    """Scalar-scale attention computed the folded way (vLLM pull request
    52060, "Suggested Fix"): the K scale multiplies the score scale, the raw
    codes are attended, and the V scale multiplies the normalized output
    once.  Used only to pin that the fold equals the plain definition."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(DIM)
    ks = float(np.asarray(k_scale).reshape(-1)[0])
    vs = float(np.asarray(v_scale).reshape(-1)[0])
    raw = attention_ref(q, k_cache, v_cache, None, None, block_table, context_lens,
                        cu_seqlens_q, sparse_page_idx, NONE, num_kv_heads,
                        sm_scale=sm_scale * ks)
    return raw * vs


# ---------------------------------------------------------------------------
# Split-K form: partial results over a subset of tokens, and their merge.
# ROCm/ATOM pull request 2710 review ("Must fix" 1) names the per-partition
# scratch -- a running max, a running sum and an unnormalized accumulator
# per (KV head, row) -- and ROCm/ATOM pull request 2614's follow-up names
# split-K as the missing piece.  The merge is the log-sum-exp combination.

def attention_partial(qv, k, v, sm_scale):
    """(m, l, acc) of one query vector over a token subset, natural exp.
    An empty subset gives (-inf, 0, 0)."""
    if k.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(DIM)
    s = sm_scale * (k @ qv)
    m = float(s.max())
    w = np.exp(s - m)
    return m, float(w.sum()), w @ v


def lse_merge(partials):
    """Combine (m, l, acc) partials into the normalized output (0 if all empty)."""
    ms = np.array([p[0] for p in partials], dtype=np.float64)
    if len(ms) == 0 or np.all(np.isneginf(ms)):
        return np.zeros(DIM)
    M = ms.max()
    w = np.exp(ms - M)
    num = sum(wi * p[2] for wi, p in zip(w, partials))
    den = sum(wi * p[1] for wi, p in zip(w, partials))
    return num / den


# ---------------------------------------------------------------------------
# Brute force: loops over every attended (token, dim) with scalar decode and
# scalar index functions and exactly rounded sums.  Tiny inputs only.

def attention_bruteforce(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                         cu_seqlens_q=None, sparse_page_idx=None, mode=PER_TOKEN,
                         num_kv_heads=1, sm_scale=None, kv_dtype="fp8"):
    q = np.asarray(q, dtype=np.float64)
    rows = q.shape[0]
    Hkv = num_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(DIM)
    block_table = np.asarray(block_table)
    B, W = block_table.shape
    num_blocks = k_cache.size // (Hkv * PAGE * DIM)
    # request of each row, by walking the row ranges
    if cu_seqlens_q is None:
        L = rows // B
        starts = [b * L for b in range(B + 1)]
    else:
        starts = [int(x) for x in cu_seqlens_q]
    out = np.zeros((rows, GROUP * Hkv, DIM))
    for b in range(B):
        Lb = starts[b + 1] - starts[b]
        for i in range(Lb):
            r = starts[b] + i
            limit = min(int(context_lens[b]) - Lb + i + 1, W * PAGE)
            if sparse_page_idx is None:
                toks = list(range(max(limit, 0)))
            else:
                toks = []
                for n in sparse_page_idx[r]:
                    n = int(n)
                    if n < 0 or n >= W:
                        continue
                    toks += [t for t in range(n * PAGE, (n + 1) * PAGE) if t < limit]
            for h in range(Hkv):
                kv = []
                for t in toks:
                    P = int(block_table[b, t // PAGE])
                    if P < 0 or P >= num_blocks:
                        continue
                    o = t % PAGE
                    base = (P * Hkv + h) * PAGE * DIM
                    if kv_dtype == "bf16":
                        sk = sv = 1.0
                    elif mode == PER_TOKEN:
                        sk = float(k_scale[(P * Hkv + h) * PAGE + o])
                        sv = float(v_scale[(P * Hkv + h) * PAGE + o])
                    elif mode == SCALAR:
                        sk, sv = float(k_scale[0]), float(v_scale[0])
                    else:
                        sk = sv = 1.0
                    if kv_dtype == "bf16":
                        kvec = [float(bf16.decode(k_cache[base + int(layout.k_offset_bf16(o, d))]))
                                for d in range(DIM)]
                        vvec = [float(bf16.decode(v_cache[base + int(layout.v_offset_bf16(o, d))]))
                                for d in range(DIM)]
                    else:
                        kvec = [e4m3.decode_byte(k_cache[base + int(layout.k_offset(o, d))]) * sk
                                for d in range(DIM)]
                        vvec = [e4m3.decode_byte(v_cache[base + int(layout.v_offset(o, d))]) * sv
                                for d in range(DIM)]
                    kv.append((kvec, vvec))
                for j in range(GROUP):
                    qh = q[r, GROUP * h + j]
                    if not kv:
                        continue
                    scores = [sm_scale * math.fsum(qh[d] * kvec[d] for d in range(DIM))
                              for kvec, _ in kv]
                    mx = max(scores)
                    ws = [math.exp(s - mx) for s in scores]
                    den = math.fsum(ws)
                    for d in range(DIM):
                        out[r, GROUP * h + j, d] = math.fsum(
                            w * vvec[d] for w, (_, vvec) in zip(ws, kv)) / den
    return out
