"""GPU tests of pa_check_decode_inputs: the device-side check of a decode
call's inputs.  Well-formed calls of every kind report nothing; each
precondition violation, planted from the host in the device tensors,
reports its kind and its first offending index; a fault in what the call
does not read (a table entry or scale past the context) is not reported."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase

pytestmark = pytest.mark.gpu

CLEAN = [
    dict(seed=301, ctx=[300, 513], q_lens=[1, 1]),
    dict(seed=302, ctx=[900, 260, 131, 4], q_lens=[4, 4, 4, 4], Hkv=2),
    dict(seed=303, ctx=[600, 301, 250, 90], q_lens=[4, 4, 6, 2], ragged=True),
    dict(seed=304, ctx=[5000, 2100], q_lens=[1, 1], sparse_topk=6),
    dict(seed=305, ctx=[4000, 2500], q_lens=[2, 1], ragged=True, sparse_topk=5),
    dict(seed=306, ctx=[1500, 800], q_lens=[1, 1], mode=wl.SCALAR),
    dict(seed=307, ctx=[640, 129], q_lens=[2, 2], mode=wl.NONE),
]


def run_check(case):
    report = torch.full((16,), -5, dtype=torch.int32, device=case.dev)
    pa.pa_check_decode_inputs(case.q, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt, case.ctx, case.cu,
                              case.sp, case.mode, case.out, report)
    torch.cuda.synchronize()
    return pa.check_report(report)


@pytest.mark.parametrize("kw", CLEAN, ids=[str(c["seed"]) for c in CLEAN])
def test_well_formed_calls_report_nothing(kw):
    w = wl.small_case(**kw)
    print("check clean case", w.name, flush=True)
    r = run_check(GpuCase(w))
    assert r == {"count": 0, "kinds": [], "first": {}}, r


def test_bf16_cache_call_reports_nothing():
    w = wl.bf16_kv(wl.small_case(seed=308, ctx=[700, 45], q_lens=[1, 1]))
    r = run_check(GpuCase(w))
    assert r["count"] == 0, r


def test_cu_seqlens_violations():
    w = wl.small_case(seed=309, ctx=[600, 301, 250, 90], q_lens=[4, 4, 6, 2], ragged=True)
    case = GpuCase(w)
    cu = w.cu.copy()
    cu[2] = cu[1] - 1  # request 1 ends before it starts
    case.cu.copy_(torch.from_numpy(cu))
    r = run_check(case)
    assert "cu_order" in r["kinds"] and r["first"]["cu_order"] == 1, r
    assert "cu_ends" not in r["kinds"], r
    cu = w.cu.copy()
    cu[-1] = w.rows - 1  # the last request claims one row fewer than q holds
    case.cu.copy_(torch.from_numpy(cu))
    r = run_check(case)
    assert r["kinds"] == ["cu_ends"] and r["first"]["cu_ends"] == 0, r


def test_context_shorter_than_q_len():
    w = wl.small_case(seed=310, ctx=[900, 260, 131, 40], q_lens=[4, 4, 4, 4])
    case = GpuCase(w)
    ctx = w.ctx.copy()
    ctx[2] = 3
    case.ctx.copy_(torch.from_numpy(ctx))
    r = run_check(case)
    assert "ctx_short" in r["kinds"] and r["first"]["ctx_short"] == 2, r


def test_block_table_ids_of_attended_pages_only():
    w = wl.small_case(seed=311, ctx=[1000, 300], q_lens=[1, 1], W=12)
    case = GpuCase(w)
    # past request 1's context (300 tokens = 3 pages): never read, not reported
    bt = w.block_table.copy()
    bt[1, 8] = w.num_blocks + 100
    case.bt.copy_(torch.from_numpy(bt))
    assert run_check(case)["count"] == 0
    bt[0, 5] = w.num_blocks + 7   # attended: out of the pool
    bt[1, 2] = -3                 # attended: negative
    case.bt.copy_(torch.from_numpy(bt))
    r = run_check(case)
    assert r["kinds"] == ["table_id"] and r["count"] == 2, r
    assert r["first"]["table_id"] == 0 * w.W + 5, r


def test_sparse_list_violations():
    w = wl.small_case(seed=312, ctx=[5000, 2100], q_lens=[1, 1], sparse_topk=6)
    case = GpuCase(w)
    sp = w.sparse.copy()
    sp[1, 3] = w.W + 3       # not a logical page
    sp[0, 4] = sp[0, 1]      # listed twice
    sp[1, 5] = -1            # padding: fine
    case.sp.copy_(torch.from_numpy(sp))
    r = run_check(case)
    assert set(r["kinds"]) == {"sparse_id", "sparse_dup"}, r
    assert r["first"]["sparse_id"] == 1 * 6 + 3 and r["first"]["sparse_dup"] == 0, r


def test_per_token_scales_of_attended_tokens_only():
    w = wl.small_case(seed=313, ctx=[300, 513], q_lens=[1, 1])
    case = GpuCase(w)
    ks = case.ks.view(-1, w.Hkv, 128)
    vs = case.vs.view(-1, w.Hkv, 128)
    P = int(w.block_table[0, 2])  # request 0's last page holds tokens 256..299
    ks[P, 0, 60] = float("nan")   # slot 60 = token 316, past the context: not reported
    assert run_check(case)["count"] == 0
    vs[P, 0, 10] = -1.0           # token 266: attended
    P1 = int(w.block_table[1, 1])
    ks[P1, 0, 5] = float("inf")   # request 1, page 1
    r = run_check(case)
    assert r["kinds"] == ["scale"] and r["count"] == 2, r
    assert r["first"]["scale"] == 0 * w.W + 2, r


@pytest.mark.parametrize("bad", [0.0, float("inf"), float("nan")])
def test_scalar_scale(bad):
    w = wl.small_case(seed=314, ctx=[1500, 800], q_lens=[1, 1], mode=wl.SCALAR)
    case = GpuCase(w)
    case.vs_arg.fill_(bad)
    r = run_check(case)
    assert r["kinds"] == ["scale"] and r["first"]["scale"] == 0, r


def test_report_is_reset_on_each_call():
    w = wl.small_case(seed=315, ctx=[1000, 300], q_lens=[1, 1])
    case = GpuCase(w)
    report = torch.full((16,), 0, dtype=torch.int32, device=case.dev)
    bt = w.block_table.copy()
    bt[0, 1] = -1
    case.bt.copy_(torch.from_numpy(bt))
    pa.pa_check_decode_inputs(case.q, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt, case.ctx, None, None,
                              case.mode, case.out, report)
    torch.cuda.synchronize()
    assert pa.check_report(report)["count"] == 1
    case.bt.copy_(torch.from_numpy(w.block_table))
    pa.pa_check_decode_inputs(case.q, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt, case.ctx, None, None,
                              case.mode, case.out, report)
    torch.cuda.synchronize()
    assert pa.check_report(report) == {"count": 0, "kinds": [], "first": {}}
    assert np.all(report.cpu().numpy()[2:9] == np.iinfo(np.int32).max)
