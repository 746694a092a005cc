"""GPU parity of the prefill kernel: calls whose requests hold at least 128
query rows, with that length known to the host (uniform q_len, or
max_q_len), run a kernel whose workgroups own 8 consecutive positions of a
request and share each K/V chunk through LDS.  Row i of a q_len-L request
still sees context_len - L + i + 1 tokens (ROCm/ATOM pull request 2122,
section 2), so every case is checked element by element against the fp64
oracle (decode tolerance: max|err| <= 1e-2 where |ref| < 4, 2^-7|ref| above,
cosine >= 0.9999), and against the decode kernel on the same call (an
explicitly balanced split keeps the decode kernel) to 4e-3.

Cases: prompts whose length is not a multiple of the 8-position group (a
last group with one position, waves with no rows), a chunked prefill over
an earlier context, ragged segments of mixed lengths, two KV heads, the
scalar and no-scale modes, forced partitions (partials through the merge
kernel), uniform q_len without cu_seqlens_q, a segment whose page table
entries are permuted over a poisoned pool, and the unquantized bf16 cache
(whose poison includes NaN and infinity patterns past the context)."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_cache, oracle_out

pytestmark = pytest.mark.gpu

CASES = [
    dict(seed=501, ctx=[300], q_lens=[300], ragged=True),                 # a prompt, 37.5 groups
    dict(seed=502, ctx=[257], q_lens=[257], ragged=True, Hkv=2),          # last group: one position
    dict(seed=503, ctx=[1000], q_lens=[128], ragged=True),                # chunked prefill over 872 tokens
    dict(seed=504, ctx=[140, 500, 100, 700], q_lens=[140, 33, 100, 1], ragged=True),  # mixed lengths
    dict(seed=505, ctx=[200, 333], q_lens=[130, 130]),                    # uniform, no cu_seqlens_q
    dict(seed=506, ctx=[190, 650], q_lens=[190, 35], ragged=True, mode=wl.SCALAR),
    dict(seed=507, ctx=[129, 400], q_lens=[129, 40], ragged=True, mode=wl.NONE),
]


def _config(w):
    mq = int(w.q_lens.max())
    return pa.make_config(w.Hkv, w.rows, w.B, w.W, ragged=w.cu is not None,
                          max_q_len=mq if w.cu is not None else 0, scale_mode=w.mode)


def _run(case, w, **kw):
    mq = int(w.q_lens.max()) if w.cu is not None else 0
    out = case.decode(out=torch.empty_like(case.out), max_q_len=mq, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kw", CASES, ids=[str(c["seed"]) for c in CASES])
def test_prefill_kernel_against_oracle(kw):
    w = wl.small_case(**kw)
    plan = pa.pa_plan_describe(_config(w))
    assert plan["rows_per_group"] == 8, plan          # the prefill kernel
    print("prefill kernel case", w.name, "rows", w.rows, "plan", plan["groups"], plan["parts"], flush=True)
    case = GpuCase(w)
    ref = oracle_out(w, oracle_cache(w))
    out = _run(case, w)
    compare(out, ref, what=f"{w.name} prefill kernel")
    # the decode kernel on the same call
    dec = _run(case, w, partition_mode=pa.PARTITION_BALANCED) if w.B <= 64 else None
    if dec is not None:
        compare(out, dec.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{w.name} vs decode kernel")
    # forced partitions: partials of the page ranges, merged by the merge kernel
    for parts in (2, 3, 7):
        print("  force_parts", parts, flush=True)
        o = _run(case, w, force_parts=parts)
        compare(o, ref, what=f"{w.name} prefill kernel, {parts} partitions")


def test_prefill_kernel_permuted_pages_bitwise():
    """Permuting the physical pages through the block table (and moving the
    bytes with them) leaves the output bitwise unchanged."""
    w = wl.small_case(seed=508, ctx=[600], q_lens=[600], ragged=True)
    case = GpuCase(w)
    out1 = _run(case, w)
    perm = np.random.default_rng(509).permutation(w.num_blocks)
    # page p moves to perm[p]
    kc = torch.empty_like(case.kc)
    vc = torch.empty_like(case.vc)
    ks = torch.empty_like(case.ks)
    vs = torch.empty_like(case.vs)
    pt = torch.from_numpy(perm).to(case.dev)
    kc[pt] = case.kc
    vc[pt] = case.vc
    ks[pt] = case.ks
    vs[pt] = case.vs
    case.kc, case.vc, case.ks, case.vs = kc, vc, ks, vs
    case.ks_arg, case.vs_arg = ks, vs
    bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    case.bt = torch.from_numpy(bt).to(case.dev)
    out2 = _run(case, w)
    assert torch.equal(out1, out2)


def test_prefill_16k_kernel_rows_sampled():
    """The 16384-token prompt (the size the pages give) on the prefill
    kernel, sampled rows against the oracle, every row finite."""
    T = 16384
    w = wl.small_case(seed=510, ctx=[T], q_lens=[T], ragged=True)
    plan = pa.pa_plan_describe(_config(w))
    assert plan["rows_per_group"] == 8 and plan["parts"] == 1, plan
    case = GpuCase(w)
    out = _run(case, w)
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g))
    rng = np.random.default_rng(511)
    rows = sorted(set([0, 1, 7, 8, 127, 128, 8191, 8192, T - 9, T - 8, T - 1] +
                      [int(x) for x in rng.integers(0, T, size=10)]))
    ref = oracle_out(w, oracle_cache(w), rows_subset=rows)
    compare(g[rows], ref, what="prefill kernel 16K")


BF16_CASES = [
    dict(seed=521, ctx=[300], q_lens=[300], ragged=True),
    dict(seed=522, ctx=[700, 257], q_lens=[150, 257], ragged=True, Hkv=2),
    dict(seed=523, ctx=[200, 333], q_lens=[130, 130]),
]


@pytest.mark.parametrize("kw", BF16_CASES, ids=[str(c["seed"]) for c in BF16_CASES])
def test_prefill_kernel_bf16_cache(kw):
    w = wl.bf16_kv(wl.small_case(**kw))
    cfg = pa.make_config(w.Hkv, w.rows, w.B, w.W, ragged=w.cu is not None,
                         max_q_len=int(w.q_lens.max()) if w.cu is not None else 0,
                         scale_mode=wl.NONE, kv_dtype=3)  # bf16
    assert pa.pa_plan_describe(cfg)["rows_per_group"] == 8
    print("prefill kernel bf16 case", w.name, flush=True)
    case = GpuCase(w)
    ref = oracle_out(w)
    out = _run(case, w)
    compare(out, ref, what=f"{w.name} prefill kernel")
    dec = _run(case, w, partition_mode=pa.PARTITION_BALANCED)
    compare(out, dec.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{w.name} vs decode kernel")
    for parts in (2, 5):
        compare(_run(case, w, force_parts=parts), ref, what=f"{w.name} prefill kernel, {parts} partitions")
