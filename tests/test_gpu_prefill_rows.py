"""Per-token-as-decode prefill (prompt tokens pushed through the decode
contract as rows; ROCm/ATOM pull request 2614, "Change", reuses the decode
contract for per-token-as-decode prefill) and other wide-row shapes: many
KV heads, long q_len split into several row groups, rows near the capacity
buckets.  Every case is checked element by element against the oracle."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_cache, oracle_out

pytestmark = pytest.mark.gpu


def _as_token_rows(w):
    """The same prompt as T requests of q_len 1: row t is its own request with
    context t+1 (counting itself) and the prompt's block table."""
    T = int(w.ctx[0])
    bt = np.repeat(w.block_table[:1], T, axis=0)
    return bt, np.arange(1, T + 1, dtype=np.int32)


@pytest.mark.parametrize("T,Hkv", [(300, 1), (257, 2)])
def test_prompt_as_decode_rows_equals_causal_prefill(T, Hkv):
    # one request whose q_len is the whole prompt (ragged form), and the same
    # prompt as T single-row requests: both must match the oracle
    w = wl.small_case(seed=301 + T, ctx=[T], q_lens=[T], Hkv=Hkv, ragged=True)
    case = GpuCase(w)
    out_multi = case.decode(out=torch.empty_like(case.out), max_q_len=T).clone()
    torch.cuda.synchronize()
    cache = oracle_cache(w)
    ref = oracle_out(w, cache)
    compare(out_multi, ref, what=f"prefill as one request q_len {T}")

    bt, ctx = _as_token_rows(w)
    out_rows = torch.empty_like(case.out)
    pa.pa_decode(case.q, case.kc, case.vc, case.ks_arg, case.vs_arg, torch.from_numpy(bt).to(case.dev),
                 torch.from_numpy(ctx).to(case.dev), None, None, w.mode, out_rows)
    torch.cuda.synchronize()
    compare(out_rows, ref, what=f"prefill as {T} decode rows")


@pytest.mark.parametrize("Hkv", [4, 8])
def test_many_kv_heads(Hkv):
    w = wl.small_case(seed=320 + Hkv, ctx=[700, 129, 5], q_lens=[2, 2, 2], Hkv=Hkv)
    case = GpuCase(w)
    for parts in (0, 1, 5):
        out = case.decode(out=torch.empty_like(case.out), force_parts=parts) if parts else \
            case.decode(out=torch.empty_like(case.out))
        torch.cuda.synchronize()
        compare(out, oracle_out(w), what=f"Hkv {Hkv} parts {parts}")


def test_uniform_q_len_8_uses_row_groups():
    w = wl.small_case(seed=330, ctx=[600, 300, 1000], q_lens=[8, 8, 8])
    cfg = pa.make_config(1, w.rows, w.B, w.W)
    plan = pa.pa_plan_describe(cfg)
    assert plan["rows_per_group"] == 2 and plan["groups"] == 4
    case = GpuCase(w)
    out = case.decode()
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what="q_len 8")


def test_sparse_ragged_scalar_none_mix():
    for mode in (wl.SCALAR, wl.NONE):
        w = wl.small_case(seed=340 + mode, ctx=[3000, 2600, 1400], q_lens=[3, 1, 2], ragged=True,
                          sparse_topk=5, mode=mode)
        w.sparse[2, 4] = -1
        case = GpuCase(w)
        for parts in (0, 2):
            out = case.decode(out=torch.empty_like(case.out), force_parts=parts) if parts else \
                case.decode(out=torch.empty_like(case.out))
            torch.cuda.synchronize()
            compare(out, oracle_out(w), what=f"sparse ragged mode {mode} parts {parts}")


def test_rows_across_capacity_buckets():
    """Row counts on both sides of power-of-two buckets reuse the same
    reserved scratch; results stay exact."""
    rng = np.random.default_rng(350)
    for B in (31, 32, 33, 64, 65):
        ctx = rng.integers(1, 700, size=B)
        w = wl.small_case(seed=350 + B, ctx=list(ctx), q_lens=[1] * B)
        case = GpuCase(w)
        out = case.decode()
        torch.cuda.synchronize()
        compare(out, oracle_out(w), what=f"batch {B}")
