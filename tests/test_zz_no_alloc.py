"""pa_decode_noalloc: the decode entry point that allocates nothing (its
split-K partials live in the library's fixed device array).  Its results
equal pa_decode_ex's on the same inputs -- same kernels, same plan -- over
two calls in a row (the second smaller, so it reads the array the first one
left behind), and under graph capture with nothing reserved.  Calls whose
scratch bucket exceeds the array, or that ask for the in-kernel merge, are
refused before launch."""

import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_out

pytestmark = pytest.mark.gpu

CAPACITY, UNSUPPORTED = -6, -5
MAX_BYTES = 32 << 20


def _noalloc(case, out, **kw):
    w = case.w
    return pa.pa_decode_noalloc(case.q, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt, case.ctx,
                                case.cu, case.sp, w.mode, out, **kw)


def _pair(case, **kw):
    ref = case.decode(out=torch.empty_like(case.out), **kw)
    got = _noalloc(case, torch.full_like(case.out, 3.0), **kw)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), kw
    return got


def test_two_calls_second_smaller():
    big = wl.small_case(seed=961, ctx=[9000, 5000, 4000, 2000, 300, 129], q_lens=[2, 1, 3, 1, 1, 2],
                        ragged=True)
    small = wl.small_case(seed=962, ctx=[700, 1500], q_lens=[1, 1])
    cb, cs = GpuCase(big), GpuCase(small)
    print("noalloc: big, then small", flush=True)
    for kw in (dict(max_q_len=3), dict(max_q_len=3, force_parts=40)):
        got = _pair(cb, **kw)
        compare(got, oracle_out(big), what=f"noalloc big {kw}")
    for kw in (dict(), dict(force_parts=5)):
        got = _pair(cs, **kw)
        compare(got, oracle_out(small), what=f"noalloc small {kw}")


@pytest.mark.parametrize("kind", ["sparse", "balanced_q4", "scalar", "c2"])
def test_plans_match_pa_decode_ex(kind):
    if kind == "sparse":
        w = wl.small_case(seed=963, ctx=[3000, 2600, 1400], q_lens=[3, 1, 2], ragged=True, sparse_topk=5)
        kws = [dict(max_q_len=3), dict(max_q_len=3, force_parts=2)]
    elif kind == "balanced_q4":
        w = wl.small_case(seed=964, ctx=[3000, 1200, 70, 5000], q_lens=[4, 4, 4, 4])
        kws = [dict(), dict(partition_mode=pa.PARTITION_BALANCED)]
    elif kind == "scalar":
        w = wl.small_case(seed=965, ctx=[4000, 513], q_lens=[1, 1], mode=wl.SCALAR, Hkv=2)
        kws = [dict(), dict(force_parts=7)]
    else:
        w = wl.c2_dense_8k()
        kws = [dict()]
    case = GpuCase(w)
    print("noalloc plans", kind, flush=True)
    for kw in kws:
        _pair(case, **kw)


def test_refusals_before_launch():
    w = wl.small_case(seed=966, ctx=[600, 300], q_lens=[1, 1])
    case = GpuCase(w)
    out = torch.full_like(case.out, 5.0)
    with pytest.raises(pa.PaError) as ei:
        _noalloc(case, out, force_parts=4, merge_mode=pa.MERGE_IN_KERNEL)
    assert ei.value.status == UNSUPPORTED
    # 16K single-row requests of 8 partitions each: a scratch bucket above the array
    T = 16384
    cfg = pa.make_config(1, T, T, w.W, force_parts=8)
    assert pa.pa_plan_describe(cfg)["scratch_bytes"] > MAX_BYTES
    q = torch.zeros(T, 16, 128, dtype=torch.bfloat16, device=case.dev)
    o = torch.full((T, 16, 128), 5.0, dtype=torch.bfloat16, device=case.dev)
    bt = case.bt[:1].repeat(T, 1)
    ctx = case.ctx[:1].repeat(T)
    with pytest.raises(pa.PaError) as ei:
        pa.pa_decode_noalloc(q, case.kc, case.vc, case.ks_arg, case.vs_arg, bt, ctx, None, None, w.mode, o,
                             force_parts=8)
    assert ei.value.status == CAPACITY
    assert "pa_decode_noalloc" in pa.pa_last_error()
    torch.cuda.synchronize()
    assert torch.all(out.float() == 5.0) and torch.all(o.float() == 5.0)


def test_capture_with_nothing_reserved():
    """Under capture on a fresh stream (no arena, nothing reserved) the call
    records and replays; replays with eager work between them match eager."""
    w = wl.small_case(seed=967, ctx=[3000, 1200, 700], q_lens=[1, 1, 1])
    case = GpuCase(w)
    eager = case.decode(out=torch.empty_like(case.out), force_parts=6)
    _noalloc(case, torch.empty_like(case.out), force_parts=6)   # first call on the device: outside capture
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    out = torch.empty_like(case.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        _noalloc(case, out, force_parts=6)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        other = _noalloc(case, torch.empty_like(case.out), force_parts=3)
        torch.cuda.synchronize()
        compare(other, oracle_out(w), what=f"eager between replays {rep}")
    compare(eager, oracle_out(w), what="eager")
