"""Seeded synthetic inputs for paged FP8-KV decode attention.

Shared by the tests, the bench and the oracle checks.  This module draws
random numbers and lays out shapes only; it holds none of the method's
arithmetic (no quantization, no attention, no cache layout).

Every value is a pure function of (workload seed, what it is): the K/V
values of logical page n of request b come from their own generator seeded
with (seed, b, n), so any page can be regenerated alone -- large workloads
check sampled rows without materialising the whole context on the host.

Shapes follow the pages' serving workloads: 128-token pages (vLLM serve
flag --block-size 128), 16 query heads per KV head and head dim 128
(query view [requests, q_len, 1, 16, 128]), q_len 4 for three speculative
tokens plus one, batch 4 (concurrency) for 8K contexts and 32
(--max-num-seqs) for 128K contexts.
"""

from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

PAGE = 128
DIM = 128
GROUP = 16
NONE, SCALAR, PER_TOKEN = 0, 1, 2


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32.
    Input preparation for the bf16 query tensor."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def rope_tables(max_pos: int, rot: int, base: float = 10000.0):
    """Cosine and sine tables [max_pos, rot/2] (fp32) of the usual rotary
    frequencies: column i turns by base^(-2i/rot) radians per position.
    Model parameters handed to the fused writer, computed in fp64 and rounded
    once to fp32."""
    i = np.arange(rot // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / rot)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hkv: int
    rows: int
    ctx: np.ndarray                      # int32 [B]
    q_lens: np.ndarray                   # int32 [B]
    cu: Optional[np.ndarray]             # int32 [B+1] or None (uniform)
    block_table: np.ndarray              # int32 [B, W]
    num_blocks: int
    sparse: Optional[np.ndarray] = None  # int32 [rows, topk] logical pages or None
    mode: int = PER_TOKEN
    k_scalar: float = 1.0
    v_scalar: float = 1.0
    written: List[np.ndarray] = field(default_factory=list)  # per request: logical pages holding data
    q: Optional[np.ndarray] = None       # float32 (bf16-exact) [rows, 16*Hkv, 128]
    sm_scale: Optional[float] = None
    kv_dtype: str = "fp8"                # "fp8" (e4m3fn codes) or "bf16" (unquantized)

    @property
    def W(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def Hq(self) -> int:
        return GROUP * self.Hkv

    @property
    def row_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int64)

    def page_kv(self, b: int, n: int):
        """fp32 K and V of the valid tokens of logical page n of request b:
        two arrays [cnt, Hkv, 128] drawn N(0,1), cnt = tokens of that page
        inside the context."""
        cnt = int(min(PAGE, int(self.ctx[b]) - n * PAGE))
        g = np.random.default_rng([self.seed, 7, b, n])
        k = g.standard_normal((cnt, self.Hkv, DIM), dtype=np.float32)
        v = g.standard_normal((cnt, self.Hkv, DIM), dtype=np.float32)
        return k, v

    def page_slots(self, b: int, n: int) -> np.ndarray:
        cnt = int(min(PAGE, int(self.ctx[b]) - n * PAGE))
        P = int(self.block_table[b, n])
        return (P * PAGE + np.arange(cnt)).astype(np.int64)

    def request_kv(self, b: int, pages=None):
        """Concatenated (k, v, slots) of the written pages of request b."""
        pages = self.written[b] if pages is None else pages
        ks, vs, ss = [], [], []
        for n in pages:
            k, v = self.page_kv(b, int(n))
            ks.append(k)
            vs.append(v)
            ss.append(self.page_slots(b, int(n)))
        if not ks:
            z = np.zeros((0, self.Hkv, DIM), np.float32)
            return z, z.copy(), np.zeros(0, np.int64)
        return np.concatenate(ks), np.concatenate(vs), np.concatenate(ss)

    def step_tokens(self):
        """The decode step's own new tokens: the last q_len tokens of every
        request, as (k, v, slots) with one entry per query row."""
        ks, vs, ss = [], [], []
        for b in range(self.B):
            L = int(self.q_lens[b])
            c = int(self.ctx[b])
            for t in range(c - L, c):
                n, o = divmod(t, PAGE)
                k, v = self.page_kv(b, n)
                ks.append(k[o])
                vs.append(v[o])
                ss.append(int(self.block_table[b, n]) * PAGE + o)
        return (np.stack(ks) if ks else np.zeros((0, self.Hkv, DIM), np.float32),
                np.stack(vs) if vs else np.zeros((0, self.Hkv, DIM), np.float32),
                np.asarray(ss, dtype=np.int64))

    # ---- sparse-indexer inputs (index keys and index queries) -------------
    def index_page_codes(self, b: int, n: int) -> np.ndarray:
        """uint8 [cnt, 128] index-key codes of the valid tokens of logical
        page n of request b: random sign, magnitude code uniform in
        [0x28, 0x40) (e4m3fn magnitudes 0.25 .. 1.875).  Random bytes only."""
        cnt = int(min(PAGE, int(self.ctx[b]) - n * PAGE))
        g = np.random.default_rng([self.seed, 11, b, n])
        mag = g.integers(0x28, 0x40, size=(cnt, DIM), dtype=np.uint8)
        sign = g.integers(0, 2, size=(cnt, DIM), dtype=np.uint8) << 7
        return mag | sign

    def index_queries(self) -> np.ndarray:
        """float32 (bf16-exact) [rows, 128] index queries."""
        g = np.random.default_rng([self.seed, 13])
        return bf16_round(g.standard_normal((self.rows, DIM), dtype=np.float32))

    def index_cache(self, poison: bool = True, num_blocks: Optional[int] = None,
                    page_map=None) -> np.ndarray:
        """Flat uint8 index cache of shape (num_blocks, 128, 128), token-major:
        every page of every context filled, the rest random bytes (NaN codes
        included) or zero.  page_map: optional {(b, n): physical page} to
        build a compact cache instead of using the block table."""
        nb = self.num_blocks if num_blocks is None else num_blocks
        if poison:
            cache = np.random.default_rng([self.seed, 17]).integers(0, 256, size=nb * PAGE * DIM,
                                                                     dtype=np.uint8)
        else:
            cache = np.zeros(nb * PAGE * DIM, np.uint8)
        view = cache.reshape(nb, PAGE, DIM)
        for b in range(self.B):
            npages = min((int(self.ctx[b]) + PAGE - 1) // PAGE, self.W)
            for n in range(npages):
                P = int(self.block_table[b, n]) if page_map is None else page_map.get((b, n), -1)
                if 0 <= P < nb:
                    codes = self.index_page_codes(b, n)
                    view[P, :codes.shape[0]] = codes
        return cache

    def kv_bytes_attended(self) -> int:
        """Algorithmic KV bytes one decode call must read: every distinct
        (request, KV head, attended token) once, 256 code bytes plus 8 scale
        bytes in per-token mode (512 bytes for a bf16 cache)."""
        if self.kv_dtype == "bf16":
            return self.attended_tokens() * self.Hkv * 4 * DIM
        per_tok = 2 * DIM + (8 if self.mode == PER_TOKEN else 0)
        return self.attended_tokens() * self.Hkv * per_tok

    def attended_tokens(self) -> int:
        """Distinct attended tokens summed over requests (one KV head)."""
        tot = 0
        rs = self.row_start
        for b in range(self.B):
            c = int(self.ctx[b])
            if self.sparse is None:
                tot += max(0, min(c, self.W * PAGE))
            else:
                pages = set()
                for r in range(rs[b], rs[b + 1]):
                    pages |= {int(n) for n in self.sparse[r] if 0 <= n < self.W}
                for n in pages:
                    tot += max(0, min(PAGE, c - n * PAGE))
        return tot


def _make(name, seed, ctx, q_lens, Hkv, pool, ragged, mode=PER_TOKEN, W=None,
          sparse_topk=0, scalar_range=(0.01, 0.05)):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    B = len(ctx)
    need = (ctx.astype(np.int64) + PAGE - 1) // PAGE
    if W is None:
        W = int(max(1, need.max()))
    assert need.sum() <= pool, "pool too small"
    perm = rng.permutation(pool).astype(np.int32)
    bt = np.full((B, W), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    rows = int(q_lens.sum())
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32) if ragged else None
    sparse = None
    written = [np.arange(need[b]) for b in range(B)]
    if sparse_topk:
        sp = np.empty((rows, sparse_topk), dtype=np.int32)
        starts = np.concatenate([[0], np.cumsum(q_lens)])
        wr = [set() for _ in range(B)]
        for b in range(B):
            last = int(need[b]) - 1
            for r in range(starts[b], starts[b + 1]):
                pick = rng.choice(last, size=sparse_topk - 1, replace=False)
                lst = np.concatenate([pick, [last]]).astype(np.int32)
                rng.shuffle(lst)
                sp[r] = lst
                wr[b] |= set(int(x) for x in lst)
        sparse = sp
        written = [np.array(sorted(w), dtype=np.int64) for w in wr]
    Hq = GROUP * Hkv
    q = bf16_round(rng.standard_normal((rows, Hq, DIM), dtype=np.float32))
    ks = vs = 1.0
    if mode == SCALAR:
        ks = float(np.float32(rng.uniform(*scalar_range)))
        vs = float(np.float32(rng.uniform(*scalar_range)))
    return Workload(name=name, seed=seed, B=B, Hkv=Hkv, rows=rows, ctx=ctx, q_lens=q_lens,
                    cu=cu, block_table=bt, num_blocks=pool, sparse=sparse, mode=mode,
                    k_scalar=ks, v_scalar=vs, written=written, q=q)


# ---------------------------------------------------------------------------
# The five workloads (seed 20260 + index)

def c1_tiny(mode=PER_TOKEN):
    """Batch 2, q_len 1, one KV head, contexts 300 and 513 (3 + 5 pages, tails
    of 44 and 1 tokens), block table a random permutation of 8 pages."""
    return _make("c1_tiny_dense", 20261, [300, 513], [1, 1], 1, 8, False, mode)


def c2_dense_8k(mode=PER_TOKEN, seed=20262):
    """Batch 4, q_len 1, contexts uniform in [8192, 9216], 4096-page pool."""
    rng = np.random.default_rng(seed + 100000)
    ctx = rng.integers(8192, 9217, size=4)
    return _make("c2_dense_8k", seed, ctx, [1] * 4, 1, 4096, False, mode, W=72)


def c3_dense_128k(mode=PER_TOKEN):
    """Batch 32, q_len 1, context 131072 (1024 pages) each, 32768-page pool;
    scalar mode draws one K and one V scale from U[0.01, 0.05]."""
    return _make("c3_dense_128k" + ("_scalar" if mode == SCALAR else ""), 20263,
                 [131072] * 32, [1] * 32, 1, 32768, False, mode)


def c4_spec(kind="uniform"):
    """31 requests, contexts uniform in [4096, 32768].  'uniform': q_len 4
    each (124 rows); 'uniform_cu': the same with explicit cu_seqlens_q;
    'ragged': 30 x 4 rows + 1 x 1 row at a seeded position (121 rows);
    'mixed': four requests with q_lens [4, 4, 6, 2]."""
    seed = 20264
    rng = np.random.default_rng(seed + 100000)
    if kind == "mixed":
        ctx = rng.integers(4096, 32769, size=4)
        return _make("c4_spec_mixed", seed + 3, ctx, [4, 4, 6, 2], 1, 1024, True, W=256)
    ctx = rng.integers(4096, 32769, size=31)
    if kind in ("uniform", "uniform_cu"):
        return _make("c4_spec_" + kind, seed, ctx, [4] * 31, 1, 8192, kind == "uniform_cu", W=256)
    ql = np.full(31, 4)
    ql[int(rng.integers(0, 31))] = 1
    return _make("c4_spec_ragged", seed + 1, ctx, ql, 1, 8192, True, W=256)


def c5_sparse(tail=False):
    """Batch 16, q_len 1, context 131072, 16384-page pool; each row attends a
    top-32 list of pages: 31 drawn without replacement from pages 0..1022
    plus the last page, shuffled.  'tail': contexts 131072 - U{1..127} so the
    last page is partial."""
    seed = 20265
    rng = np.random.default_rng(seed + 100000)
    ctx = np.full(16, 131072)
    if tail:
        ctx = ctx - rng.integers(1, 128, size=16)
    return _make("c5_sparse" + ("_tail" if tail else ""), seed + (1 if tail else 0), ctx,
                 [1] * 16, 1, 16384, False, sparse_topk=32)


def prefill_16k(Hkv=1):
    """Per-token-as-decode prefill of a 16384-token prompt: one request whose
    q_len is the whole prompt (ragged form, cu_seqlens_q given), context
    16384 (128 pages), per-token e4m3 scales; 16384 x 16 query heads of
    bf16 output per KV head (64 MiB)."""
    return _make("prefill_16k", 20268, [16384], [16384], Hkv, 160, True)


def small_case(seed, ctx, q_lens, Hkv=1, ragged=False, mode=PER_TOKEN, sparse_topk=0,
               pool=None, W=None):
    """A parity case sized for the oracle: any contexts, q_lens and heads."""
    need = sum((int(c) + PAGE - 1) // PAGE for c in ctx)
    pool = pool or max(need + 3, 4)
    return _make(f"small_{seed}", seed, ctx, q_lens, Hkv, pool, ragged, mode, W=W,
                 sparse_topk=sparse_topk)


def bf16_kv(w: Workload) -> Workload:
    """The same workload over an unquantized bf16 cache (no scales): the
    same queries, contexts, tables and K/V draws."""
    return replace(w, name=w.name + "_bf16", kv_dtype="bf16", mode=NONE)


def index_workload(kind="c5"):
    """Sparse-indexer shapes.  'c5': the block-sparse decode shape (batch 16,
    q_len 1, context 131072, 16384-page pool) with top-32 over all 1024
    pages; 'spec': 31 requests with q_len 4, contexts in [4096, 32768],
    top-32; 'ragged': the same requests with q_lens 4 except one request of
    1 row."""
    if kind == "c5":
        w = _make("index_c5", 20266, [131072] * 16, [1] * 16, 1, 16384, False)
    else:
        rng = np.random.default_rng(20267 + 100000)
        ctx = rng.integers(4096, 32769, size=31)
        ql = np.full(31, 4)
        if kind == "ragged":
            ql[int(rng.integers(0, 31))] = 1
        w = _make("index_" + kind, 20267, ctx, ql, 1, 8192, kind == "ragged", W=256)
    return w
