"""Pins for the oracle's sparse indexer (block scores and per-row top-k)
against things other than itself: a loop-only brute force with exactly
rounded sums, the closed form for a zero query (log2 of the visible token
count), torch's own float8 decode and logsumexp for the row total,
invariance under physical page placement, and a plain sort for the top-k
rule (ties to the lower page, -inf never picked, padding)."""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import indexer as idx


def _case(seed, ctx, q_lens, ragged=False, W=None, pool=None):
    w = wl.small_case(seed=seed, ctx=ctx, q_lens=q_lens, ragged=ragged, W=W, pool=pool)
    return w, w.index_queries(), w.index_cache()


TINY = [
    dict(seed=61, ctx=[1, 5, 130], q_lens=[1, 1, 1]),
    dict(seed=62, ctx=[7, 140], q_lens=[2, 2]),
    dict(seed=63, ctx=[9, 3, 131], q_lens=[3, 1, 2], ragged=True),
]


@pytest.mark.parametrize("cfg", TINY)
def test_scores_match_bruteforce(cfg):
    w, q, cache = _case(**cfg)
    ref = idx.block_scores_ref(q, cache, w.block_table, w.ctx, w.cu)
    bru = idx.block_scores_bruteforce(q, cache, w.block_table.tolist(), w.ctx,
                                      None if w.cu is None else w.cu.tolist())
    assert np.array_equal(np.isinf(ref), np.isinf(bru))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(ref[fin], bru[fin], rtol=1e-12, atol=1e-12)


def test_zero_query_scores_are_log2_of_visible_counts():
    w, q, cache = _case(64, [300, 129], [2, 1], ragged=True)
    s = idx.block_scores_ref(np.zeros_like(q), cache, w.block_table, w.ctx, w.cu)
    # request 0 (q_len 2): rows see 299 and 300 tokens; request 1 sees 129
    want = {
        0: [7.0, 7.0, math.log2(299 - 256)],
        1: [7.0, 7.0, math.log2(300 - 256)],
        2: [7.0, 0.0, -np.inf],
    }
    for r, vals in want.items():
        np.testing.assert_allclose(s[r, :3], vals, rtol=0, atol=1e-15)


def test_row_total_matches_torch_logsumexp():
    """log2 sum_n 2^score_n equals the row's log-sum-exp over all its visible
    tokens, computed by torch from its own float8_e4m3fn decode."""
    w, q, cache = _case(65, [700, 260], [1, 3], ragged=True)
    s = idx.block_scores_ref(q, cache, w.block_table, w.ctx, w.cu)
    codes = torch.from_numpy(cache).view(torch.float8_e4m3fn).double().reshape(-1, 128, 128)
    for r in range(w.rows):
        b, i = (0, 0) if r == 0 else (1, r - 1)
        L = int(w.q_lens[b])
        lim = int(w.ctx[b]) - L + i + 1
        keys = torch.cat([codes[int(w.block_table[b, n])] for n in range((lim + 127) // 128)])[:lim]
        sc = keys @ torch.from_numpy(q[r].astype(np.float64)) / math.sqrt(128)
        want = (torch.logsumexp(sc, 0) / math.log(2.0)).item()
        fin = s[r][np.isfinite(s[r])]
        m = fin.max()
        got = m + math.log2(np.sum(np.exp2(fin - m)))
        assert abs(got - want) < 1e-12


def test_physical_placement_does_not_matter():
    w, q, cache = _case(66, [900, 400], [1, 1], pool=20)
    a = idx.block_scores_ref(q, cache, w.block_table, w.ctx)
    perm = np.random.default_rng(2).permutation(w.num_blocks)
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    view = cache.reshape(w.num_blocks, 128, 128)
    moved = np.empty_like(view)
    moved[perm] = view
    b = idx.block_scores_ref(q, moved.reshape(-1), bt2, w.ctx)
    assert np.array_equal(a, b)


def test_width_cap_and_bad_page_ids():
    w, q, _ = _case(67, [384, 200], [1, 1], W=3)
    w.ctx[0] = 1000  # past the table width: capped at 384 tokens
    cache = w.index_cache()
    w.block_table[1, 1] = w.num_blocks + 5  # outside the pool: no tokens
    s = idx.block_scores_ref(q, cache, w.block_table, w.ctx)
    capped = idx.block_scores_ref(q[:1], cache, w.block_table[:1], np.array([384]))
    assert np.array_equal(s[0], capped[0])
    assert np.all(np.isfinite(s[0, :3]))
    assert s[1, 1] == -np.inf and np.isfinite(s[1, 0])


def _topk_by_sort(scores, k):
    out = []
    for row in scores:
        cand = sorted((n for n in range(len(row)) if row[n] > -math.inf), key=lambda n: (-row[n], n))
        pick = sorted(cand[:k])
        out.append(pick + [-1] * (k - len(pick)))
    return np.array(out, dtype=np.int32)


def test_topk_matches_a_plain_sort_with_ties_and_padding():
    rng = np.random.default_rng(8)
    s = rng.integers(0, 6, size=(40, 50)).astype(np.float32)  # many ties
    s[rng.random(s.shape) < 0.2] = -np.inf
    s[3] = -np.inf
    for k in (1, 5, 17, 50, 64):
        assert np.array_equal(idx.topk_ref(s, k), _topk_by_sort(s, k)), k


def test_topk_tie_rule_by_hand():
    s = np.array([[1.0, 3.0, 3.0, -np.inf, 2.0, 3.0]])
    assert idx.topk_ref(s, 2).tolist() == [[1, 2]]
    assert idx.topk_ref(s, 4).tolist() == [[1, 2, 4, 5]]
    assert idx.topk_ref(s, 7).tolist() == [[0, 1, 2, 4, 5, -1, -1]]
