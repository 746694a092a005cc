"""GPU parity with pages past 4 GiB into the cache.

A cache on a 288 GB device can hold far more than 4 GiB per tensor, so a
(page, KV head) block's byte offset must be computed in 64 bits.  Here the
workload's pages are moved above page 140,000 of a pool sized to hold them
(K and V each ~4.6 GB), written there by kv_quant_write, and decoded; the
output must equal the oracle's on the original placement (the result does not
depend on where pages sit, which the oracle's own tests pin bitwise)."""

import copy

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import compare, oracle_out

pytestmark = pytest.mark.gpu

HIGH_BASE = 140_000  # first physical page used: 140,000 x 16 KiB x 2 heads > 4 GiB

CASES = [
    ("one-row", dict(seed=241, ctx=[1000, 300], q_lens=[1, 1], Hkv=2), False),
    ("two-row", dict(seed=242, ctx=[700, 450], q_lens=[2, 2], Hkv=2), False),
    ("sparse", dict(seed=243, ctx=[3000, 1100], q_lens=[1, 1], Hkv=2, sparse_topk=5), False),
    ("bf16", dict(seed=244, ctx=[900, 200], q_lens=[1, 1], Hkv=1), True),
]


@pytest.mark.parametrize("name,kw,bf16", CASES, ids=[c[0] for c in CASES])
def test_pages_past_4gib(name, kw, bf16):
    w = wl.small_case(**kw)
    if bf16:
        w = wl.bf16_kv(w)
    ref = oracle_out(w)
    big = copy.copy(w)
    big.block_table = (w.block_table + HIGH_BASE).astype(np.int32)
    big.num_blocks = HIGH_BASE + w.num_blocks
    elem = 2 if bf16 else 1
    assert HIGH_BASE * w.Hkv * 16384 * elem > (1 << 32)
    print("large-offset case", name, "pool pages", big.num_blocks, flush=True)
    dev = torch.device("cuda:0")
    nb, Hkv = big.num_blocks, big.Hkv
    if bf16:
        kc = torch.empty(nb, Hkv, 16384, dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        ks = vs = None
    else:
        kc = torch.empty(nb, Hkv, 16384, dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        ks = torch.empty(nb, Hkv, 128, dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
    for b in range(big.B):
        k, v, s = big.request_kv(b)
        pa.kv_quant_write(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), torch.from_numpy(s).to(dev),
                          kc, vc, ks, vs, big.mode)
    q = torch.from_numpy(big.q).to(dev).to(torch.bfloat16)
    bt = torch.from_numpy(big.block_table).to(dev)
    ctx = torch.from_numpy(big.ctx).to(dev)
    sp = None if big.sparse is None else torch.from_numpy(big.sparse).to(dev)
    for parts in (0, 1, 3):
        out = torch.empty(big.rows, big.Hq, 128, dtype=torch.bfloat16, device=dev)
        if parts:
            pa.pa_decode_ex(q, kc, vc, ks, vs, bt, ctx, None, sp, big.mode, out, force_parts=parts)
        else:
            pa.pa_decode(q, kc, vc, ks, vs, bt, ctx, None, sp, big.mode, out)
        torch.cuda.synchronize()
        compare(out, ref, what=f"{name} pages past 4 GiB parts={parts}")
    del kc, vc, ks, vs
    torch.cuda.empty_cache()


def test_index_pages_past_4gib():
    # the sparse indexer reads the fp8 index cache (num_blocks, 128, 128):
    # 16 KiB per page, so pages above 262,144 sit past 4 GiB
    from oracle import indexer as oidx
    from test_gpu_indexer import check

    base = 270_000
    w = wl.small_case(seed=245, ctx=[2000, 900], q_lens=[4, 1], ragged=True)
    print("large-offset index case, pool pages", base + w.num_blocks, flush=True)
    dev = torch.device("cuda:0")
    small = w.index_cache()
    cache = torch.empty(base + w.num_blocks, 128, 128, dtype=torch.uint8, device=dev)
    cache[base:] = torch.from_numpy(small).view(w.num_blocks, 128, 128).to(dev)
    q_np = w.index_queries()
    q = torch.from_numpy(q_np).to(dev).to(torch.bfloat16)
    bt = torch.from_numpy((w.block_table + base).astype(np.int32)).to(dev)
    ctx = torch.from_numpy(w.ctx).to(dev)
    cu = torch.from_numpy(w.cu).to(dev)
    topk = 5
    idx = torch.full((w.rows, topk), -7, dtype=torch.int32, device=dev)
    scores = torch.full((w.rows, w.W), float("nan"), dtype=torch.float32, device=dev)
    pa.pa_index_topk(q, cache, bt, ctx, cu, idx, scores)
    torch.cuda.synchronize()
    ref = oidx.block_scores_ref(q_np, small, w.block_table, w.ctx, w.cu)

    class _Case:
        pass

    c = _Case()
    c.w = w
    check(c, idx.cpu().numpy(), scores.cpu().numpy(), ref, "index pages past 4 GiB")
    del cache
    torch.cuda.empty_cache()
