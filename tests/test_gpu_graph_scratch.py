"""Split-K scratch lifetime under HIP graph capture.

The scratch arena of a (device, stream) grows when an eager call needs a
larger capacity bucket.  A graph captured before the growth keeps the old
arena's address in its kernel arguments, so the old arena must stay
allocated: replays after the growth still match the eager result bit for
bit.  A capture that would need more scratch than is reserved is refused
with PA_ERR_NOT_RESERVED and records nothing.
"""

import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_out

pytestmark = pytest.mark.gpu

NOT_RESERVED = -7


def test_replay_after_scratch_growth():
    w = wl.small_case(seed=941, ctx=[3000, 1200, 700], q_lens=[1, 1, 1])
    big = wl.small_case(seed=942, ctx=[9000, 5000, 4000, 2000, 300, 129], q_lens=[2, 1, 3, 1, 1, 2],
                        ragged=True)
    case, case_b = GpuCase(w), GpuCase(big)
    stream = torch.cuda.Stream()   # a stream of its own: its arena starts empty
    small_cfg = pa.make_config(w.Hkv, w.rows, w.B, w.W, force_parts=3)
    big_cfg = pa.make_config(big.Hkv, big.rows, big.B, big.W, ragged=True, max_q_len=3, force_parts=40)
    s_small = pa.pa_plan_describe(small_cfg)["scratch_bytes"]
    s_big = pa.pa_plan_describe(big_cfg)["scratch_bytes"]
    assert s_big > 2 * s_small, (s_small, s_big)
    pa.pa_reserve(small_cfg, stream)
    with torch.cuda.stream(stream):
        eager = case.decode(out=torch.empty_like(case.out), force_parts=3).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(case.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        case.decode(out=out, force_parts=3)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay before growth"
    for rep in range(3):
        # an eager call on the same stream that needs a larger bucket: the
        # arena grows, the one the graph holds is kept
        with torch.cuda.stream(stream):
            ob = case_b.decode(out=torch.empty_like(case_b.out), max_q_len=3, force_parts=40 + rep)
        torch.cuda.synchronize()
        compare(ob, oracle_out(big), what=f"larger bucket, eager {rep}")
        # new device allocations, filled: memory a freed arena would have
        # returned is likely to be handed out and overwritten here
        junk = [torch.full((1 << 20,), float("nan"), device="cuda:0") for _ in range(8)]
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay after growth {rep}"
        del junk
    compare(eager, oracle_out(w), what="eager")


def test_capture_without_reservation_is_refused():
    w = wl.small_case(seed=943, ctx=[2000, 900], q_lens=[1, 1])
    case = GpuCase(w)
    stream = torch.cuda.Stream()   # fresh: nothing reserved for it
    out = torch.zeros_like(case.out)
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g, stream=stream):
        out.fill_(1.0)             # the graph records this and nothing of the library
        try:
            case.decode(out=out, force_parts=4)
        except pa.PaError as e:
            status = e.status
    assert status == NOT_RESERVED, status
    assert "pa_reserve" in pa.pa_last_error()
    g.replay()
    torch.cuda.synchronize()
    assert torch.all(out.float() == 1.0), "the refused call recorded work"
    # once reserved, the same capture works and matches eager
    pa.pa_reserve(pa.make_config(w.Hkv, w.rows, w.B, w.W, force_parts=4), stream)
    g2 = torch.cuda.CUDAGraph()
    out2 = torch.empty_like(case.out)
    with torch.cuda.graph(g2, stream=stream):
        case.decode(out=out2, force_parts=4)
    g2.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        eager = case.decode(out=torch.empty_like(case.out), force_parts=4)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), eager.view(torch.int16))
    compare(eager, oracle_out(w), what="eager")
