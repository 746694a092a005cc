"""Per-token-as-decode prefill at the sizes the pages name, and the row
capacity limit.

ROCm/ATOM pull request 2614 ("Change") runs per-token FP8 prefill through
the decode contract; the review of ROCm/ATOM pull request 2710 ("Must fix"
1) sizes that path at T = 16384 prompt tokens with 16 query heads per KV
head: T * Hkv rows of work and 16384 * 16 * 128 * 2 B = 64 MiB of bf16
output per KV head.  Both forms run here at that size -- one request whose
q_len is the whole prompt, and T requests of one row each -- with sampled
rows (first, page edges, last, random) checked element by element against
the oracle, and every row checked finite.  The largest row bucket (65536
rows) is accepted and computed; one row more is refused before launch.
"""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_cache, oracle_out

pytestmark = pytest.mark.gpu

T_FULL = 16384
MAX_ROWS = 65536
CAPACITY = -6


def _sample_rows(T, rng):
    fixed = [0, 1, 126, 127, 128, 129, T // 2 - 1, T // 2, T - 129, T - 128, T - 2, T - 1]
    return sorted(set(fixed + [int(x) for x in rng.integers(0, T, size=12)]))


@pytest.mark.parametrize("Hkv", [1, 2])
def test_prefill_16k_as_one_request(Hkv):
    T = T_FULL
    w = wl.small_case(seed=360 + Hkv, ctx=[T], q_lens=[T], Hkv=Hkv, ragged=True)
    assert w.rows * w.Hq * 128 * 2 == Hkv * 64 * 2 ** 20   # 64 MiB of bf16 output per KV head
    print("prefill one request T", T, "Hkv", Hkv, flush=True)
    case = GpuCase(w)
    cfg = pa.make_config(w.Hkv, w.rows, w.B, w.W, ragged=True, max_q_len=T)
    assert pa.pa_query_support(cfg) == 0
    out = case.decode(out=torch.empty_like(case.out), max_q_len=T)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g))
    rows = _sample_rows(T, np.random.default_rng(370 + Hkv))
    ref = oracle_out(w, oracle_cache(w), rows_subset=rows)
    compare(g[rows], ref, what=f"prefill T={T} Hkv={Hkv} one request")


@pytest.mark.parametrize("Hkv", [1, 2])
def test_prefill_16k_as_decode_rows(Hkv):
    """The same prompt as T requests of q_len 1: request t has context t+1
    (counting itself) and the prompt's block table."""
    T = T_FULL
    w = wl.small_case(seed=380 + Hkv, ctx=[T], q_lens=[T], Hkv=Hkv, ragged=True)
    print("prefill decode rows T", T, "Hkv", Hkv, flush=True)
    case = GpuCase(w)
    bt = torch.from_numpy(np.repeat(w.block_table[:1], T, axis=0)).to(case.dev)
    ctx = torch.arange(1, T + 1, dtype=torch.int32, device=case.dev)
    out = torch.empty_like(case.out)
    pa.pa_decode(case.q, case.kc, case.vc, case.ks_arg, case.vs_arg, bt, ctx, None, None, w.mode, out)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g))
    rows = _sample_rows(T, np.random.default_rng(390 + Hkv))
    ref = oracle_out(w, oracle_cache(w), rows_subset=rows)   # the causal prompt: the same rows
    compare(g[rows], ref, what=f"prefill T={T} Hkv={Hkv} as decode rows")
    # and both forms agree on every row
    out1 = case.decode(out=torch.empty_like(case.out), max_q_len=T)
    torch.cuda.synchronize()
    compare(out, out1.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what="rows vs one request")


def test_row_capacity_limit():
    """65536 single-row requests (the largest row bucket) over the pages of
    64 written requests; one row more is refused with PA_ERR_CAPACITY."""
    proto = wl.small_case(seed=395, ctx=list(np.random.default_rng(395).integers(1, 1025, size=64)),
                          q_lens=[1] * 64)
    case = GpuCase(proto)
    rng = np.random.default_rng(396)
    pick = rng.integers(0, 64, size=MAX_ROWS)
    ctx = np.array([int(rng.integers(1, int(proto.ctx[p]) + 1)) for p in pick], np.int32)
    bt = proto.block_table[pick]
    q = wl.bf16_round(rng.standard_normal((MAX_ROWS, 16, 128), dtype=np.float32))
    dev = case.dev
    qt = torch.from_numpy(q).to(dev).to(torch.bfloat16)
    btt, ctt = torch.from_numpy(bt).to(dev), torch.from_numpy(ctx).to(dev)
    out = torch.empty(MAX_ROWS, 16, 128, dtype=torch.bfloat16, device=dev)
    cfg = pa.make_config(1, MAX_ROWS, MAX_ROWS, proto.W)
    assert pa.pa_query_support(cfg) == 0
    assert pa.pa_query_support(pa.make_config(1, MAX_ROWS + 1, MAX_ROWS + 1, proto.W)) == CAPACITY
    print("row capacity: 65536 rows", flush=True)
    pa.pa_decode(qt, case.kc, case.vc, case.ks_arg, case.vs_arg, btt, ctt, None, None, proto.mode, out)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g))
    cache = oracle_cache(proto)
    kc, vc, _, _, ksa, vsa = cache
    from oracle import attention as oatt
    sample = sorted(set([0, MAX_ROWS - 1] + [int(x) for x in rng.integers(0, MAX_ROWS, size=24)]))
    ref = oatt.attention_ref(q[sample], kc, vc, ksa, vsa, bt[sample], ctx[sample], None, None, proto.mode, 1)
    compare(g[sample], ref, what="65536 rows")
    # one row more: refused before anything runs, the output untouched
    q1 = torch.zeros(MAX_ROWS + 1, 16, 128, dtype=torch.bfloat16, device=dev)
    o1 = torch.full((MAX_ROWS + 1, 16, 128), 7.0, dtype=torch.bfloat16, device=dev)
    bt1 = torch.cat([btt, btt[:1]])
    ct1 = torch.cat([ctt, ctt[:1]])
    with pytest.raises(pa.PaError) as ei:
        pa.pa_decode(q1, case.kc, case.vc, case.ks_arg, case.vs_arg, bt1, ct1, None, None, proto.mode, o1)
    assert ei.value.status == CAPACITY
    torch.cuda.synchronize()
    assert torch.all(o1.float() == 7.0)
