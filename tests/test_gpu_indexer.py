"""GPU parity of pa_index_topk (the sparse indexer) against the oracle.

Block scores: every visible entry within 2e-4 + 1e-5|ref| of the fp64
oracle (an fp32 product over 128 dims and an fp32 log-sum-exp; one token
more or less in a page moves its score by ~1e-2), -inf exactly where the
oracle has it.  Page lists: exactly the top-k rule applied to the kernel's
own fp32 scores (the selection is decided in the kernel's precision), and a
valid top-k under the oracle's scores: every chosen page scores at least
as high as every page left out, up to the score tolerance.  Then the chain
indexer -> block-sparse decode against the oracle's decode of the oracle's
own lists."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl
from oracle import indexer as oidx

from harness import GpuCase, compare, oracle_out

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-4, 1e-5


class IndexCase:
    def __init__(self, w, topk, dev="cuda:0", max_q_len=0):
        self.w, self.topk, self.dev = w, topk, torch.device(dev)
        self.q_np = w.index_queries()
        self.cache_np = w.index_cache()
        self.q = torch.from_numpy(self.q_np).to(self.dev).to(torch.bfloat16)
        self.cache = torch.from_numpy(self.cache_np).to(self.dev).view(w.num_blocks, 128, 128)
        self.bt = torch.from_numpy(w.block_table).to(self.dev)
        self.ctx = torch.from_numpy(w.ctx).to(self.dev)
        self.cu = None if w.cu is None else torch.from_numpy(w.cu).to(self.dev)
        self.max_q_len = max_q_len

    def run(self, topk=None):
        k = self.topk if topk is None else topk
        idx = torch.full((self.w.rows, k), -7, dtype=torch.int32, device=self.dev)
        scores = torch.full((self.w.rows, self.w.W), float("nan"), dtype=torch.float32, device=self.dev)
        pa.pa_index_topk(self.q, self.cache, self.bt, self.ctx, self.cu, idx, scores,
                         max_q_len=self.max_q_len)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), scores.cpu().numpy()


def visible_pages(w):
    """Pages each row can see (ceil(min(limit, W*128)/128))."""
    out = []
    for b in range(w.B):
        L = int(w.q_lens[b])
        for i in range(L):
            lim = max(0, min(int(w.ctx[b]) - L + i + 1, w.W * 128))
            out.append((lim + 127) // 128)
    return out


def check(case, idx, scores, ref_scores, what):
    w = case.w
    vis = visible_pages(w)
    for r in range(w.rows):
        g, o = scores[r, :vis[r]], ref_scores[r, :vis[r]]
        assert np.array_equal(np.isinf(g), np.isinf(o)), f"{what} row {r}: -inf pattern"
        fin = np.isfinite(o)
        err = np.abs(g[fin] - o[fin])
        assert np.all(err <= ATOL + RTOL * np.abs(o[fin])), \
            f"{what} row {r}: max score err {err.max() if err.size else 0:.3e}"
    # the selection, decided in the kernel's precision
    vis_scores = np.full_like(scores, -np.inf)
    for r in range(w.rows):
        vis_scores[r, :vis[r]] = scores[r, :vis[r]]
    want = oidx.topk_ref(vis_scores, idx.shape[1])
    assert np.array_equal(idx, want), f"{what}: lists differ from the top-k of the kernel's scores"
    # valid under the oracle's scores
    for r in range(w.rows):
        chosen = idx[r][idx[r] >= 0]
        rest = np.setdiff1d(np.nonzero(np.isfinite(ref_scores[r, :vis[r]]))[0], chosen)
        if len(chosen) and len(rest):
            assert ref_scores[r, chosen].min() >= ref_scores[r, rest].max() - 2 * ATOL, f"{what} row {r}"


CASES = [
    dict(seed=501, ctx=[300, 513, 1], q_lens=[1, 1, 1]),
    dict(seed=502, ctx=[1000, 2000], q_lens=[4, 4]),                          # speculative rows
    dict(seed=503, ctx=[900, 260, 131, 4], q_lens=[4, 1, 6, 2], ragged=True),
    dict(seed=504, ctx=[3000, 40], q_lens=[20, 3], ragged=True),              # 20 rows: two 16-row groups
    dict(seed=505, ctx=[0, 700], q_lens=[1, 1]),                              # empty context
]


@pytest.mark.parametrize("kw", CASES, ids=[str(c["seed"]) for c in CASES])
@pytest.mark.parametrize("topk", [1, 3, 8, 40])
def test_index_topk_matches_oracle(kw, topk):
    w = wl.small_case(**kw)
    print("index case", w.name, "topk", topk, flush=True)
    case = IndexCase(w, topk)
    idx, scores = case.run()
    ref = oidx.block_scores_ref(case.q_np, case.cache_np, w.block_table, w.ctx, w.cu)
    check(case, idx, scores, ref, f"{w.name} topk={topk}")



def random_index_draw(seed):
    """A seeded random indexer call: batch, rows per request (uniform or
    ragged), contexts (empty, next to a page edge, or anywhere) and k."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    ragged = bool(rng.random() < 0.5)
    q_lens = [int(x) for x in rng.integers(1, 9, size=B)] if ragged else [int(rng.integers(1, 6))] * B
    ctx = []
    for L in q_lens:
        u = rng.random()
        if u < 0.1:
            c = 0
        elif u < 0.5:
            c = 128 * int(rng.integers(1, 24)) + int(rng.integers(-1, 2))
        else:
            c = int(rng.integers(1, 3000))
        ctx.append(c if c == 0 else max(c, L))
    topk = int(rng.choice([1, 2, 5, 16, 33]))
    hint = int(max(q_lens)) if ragged and rng.random() < 0.5 else 0
    return wl.small_case(seed=seed, ctx=ctx, q_lens=q_lens, ragged=ragged), topk, hint


@pytest.mark.parametrize("seed", list(range(701, 725)))
def test_random_index_calls_match_oracle(seed):
    w, topk, hint = random_index_draw(seed)
    print("random index call", seed, "q_lens", list(w.q_lens), "ctx", list(w.ctx), "topk", topk, "hint", hint,
          flush=True)
    case = IndexCase(w, topk, max_q_len=hint)
    idx, scores = case.run()
    ref = oidx.block_scores_ref(case.q_np, case.cache_np, w.block_table, w.ctx, w.cu)
    check(case, idx, scores, ref, f"random index {seed}")

def test_max_q_len_hint_gives_the_same_result():
    w = wl.small_case(seed=506, ctx=[1500, 600, 300], q_lens=[5, 1, 3], ragged=True)
    a = IndexCase(w, 6).run()
    b = IndexCase(w, 6, max_q_len=5).run()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1], equal_nan=True)


def test_width_cap_and_pages_outside_the_cache():
    w = wl.small_case(seed=507, ctx=[384, 300], q_lens=[1, 1], W=3)
    w.ctx[0] = 1000  # capped at 3 pages
    w.block_table[1, 1] = w.num_blocks + 3  # contributes no tokens
    case = IndexCase(w, 2)
    idx, scores = case.run()
    ref = oidx.block_scores_ref(case.q_np, case.cache_np, w.block_table, w.ctx)
    check(case, idx, scores, ref, "cap/outside")
    assert scores[1, 1] == -np.inf and 1 not in idx[1]


def test_chain_indexer_then_sparse_decode():
    """Lists from the GPU indexer drive the block-sparse decode; the oracle
    decodes with its own lists (asserted equal first)."""
    w = wl.small_case(seed=508, ctx=[3000, 2200, 1500], q_lens=[1, 1, 1], pool=70)
    topk = 5
    ic = IndexCase(w, topk)
    idx, scores = ic.run()
    ref_scores = oidx.block_scores_ref(ic.q_np, ic.cache_np, w.block_table, w.ctx)
    ref_lists = oidx.topk_ref(ref_scores, topk)
    assert np.array_equal(idx, ref_lists)
    w.sparse = ref_lists
    w.written = [np.arange((int(c) + 127) // 128) for c in w.ctx]
    case = GpuCase(w)
    case.sp = torch.from_numpy(idx).to(case.dev)
    out = case.decode()
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what="indexer -> sparse decode")


@pytest.mark.parametrize("kind", ["c5", "spec", "ragged"])
def test_index_full_size_sampled_rows(kind):
    w = wl.index_workload(kind)
    case = IndexCase(w, 32, max_q_len=int(w.q_lens.max()) if w.cu is not None else 0)
    idx, scores = case.run()
    assert np.all(np.isfinite(scores[:, 0]))
    # every list is the top-k of the kernel's own scores
    vis = visible_pages(w)
    vs = np.full_like(scores, -np.inf)
    for r in range(w.rows):
        vs[r, :vis[r]] = scores[r, :vis[r]]
    assert np.array_equal(idx, oidx.topk_ref(vs, 32))
    # sampled requests against the oracle
    for b in (0, w.B - 1):
        start, L = int(w.row_start[b]), int(w.q_lens[b])
        print(kind, "request", b, flush=True)
        rows = slice(start, start + L)
        ref = oidx.block_scores_ref(case.q_np[rows], case.cache_np, w.block_table[b:b + 1],
                                    w.ctx[b:b + 1], None)
        for i in range(L):
            r = start + i
            n = vis[r]
            fin = np.isfinite(ref[i, :n])
            assert np.array_equal(np.isinf(scores[r, :n]), ~fin)
            err = np.abs(scores[r, :n][fin] - ref[i, :n][fin])
            assert np.all(err <= ATOL + RTOL * np.abs(ref[i, :n][fin])), f"{kind} row {r}: {err.max():.3e}"
            chosen = idx[r][idx[r] >= 0]
            rest = np.setdiff1d(np.nonzero(fin)[0], chosen)
            assert ref[i, chosen].min() >= ref[i, rest].max() - 2 * ATOL


def test_rows_too_long_for_lds_staging():
    """A row that sees more than 8192 pages: the top-k kernel reads the
    score matrix on every pass instead of staging the keys."""
    w = wl.small_case(seed=509, ctx=[8300 * 128 - 5, 300], q_lens=[1, 1])
    print("long row case", w.W, flush=True)
    case = IndexCase(w, 64)
    idx, scores = case.run()
    ref = oidx.block_scores_ref(case.q_np, case.cache_np, w.block_table, w.ctx)
    check(case, idx, scores, ref, "8300-page row")


def test_ragged_batch_beyond_one_wave_of_requests():
    """70 ragged requests: the top-k kernel finds a row's request by binary
    search over cu_seqlens_q instead of one ballot over a wave."""
    rng = np.random.default_rng(510)
    ctx = [int(x) for x in rng.integers(1, 900, size=70)]
    q_lens = [int(x) for x in rng.integers(1, 4, size=70)]
    w = wl.small_case(seed=510, ctx=ctx, q_lens=q_lens, ragged=True)
    print("70 ragged requests", w.rows, flush=True)
    case = IndexCase(w, 3, max_q_len=3)
    idx, scores = case.run()
    ref = oidx.block_scores_ref(case.q_np, case.cache_np, w.block_table, w.ctx, w.cu)
    check(case, idx, scores, ref, "70 ragged requests")
