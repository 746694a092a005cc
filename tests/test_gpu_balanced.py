"""GPU parity of length-balanced split-K partitions (pa_partition_mode
BALANCED: one partition size per call, chosen on the device from the
context lengths; each request's partials at (slot, row within the request))
against the fp64 oracle, to the decode tolerance: single-row, multi-row,
ragged (with max_q_len), scalar, no-scale and bf16 caches, several KV heads,
context mixes from empty to long, the 64-request limit, repeated calls and
graph replays."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_out

pytestmark = pytest.mark.gpu

BAL = pa.PARTITION_BALANCED

CASES = [
    dict(seed=601, ctx=[300, 513], q_lens=[1, 1]),
    dict(seed=602, ctx=[1, 2, 127, 128, 129, 1000], q_lens=[1] * 6, Hkv=2),
    dict(seed=603, ctx=[700, 45, 300], q_lens=[2, 2, 2]),
    dict(seed=604, ctx=[900, 260, 131, 4], q_lens=[4, 4, 4, 4]),
    dict(seed=605, ctx=[600, 301, 250, 90], q_lens=[4, 4, 6, 2], ragged=True),
    dict(seed=606, ctx=[500, 40, 333], q_lens=[3, 1, 4], ragged=True, Hkv=2),
    dict(seed=607, ctx=[1500, 800], q_lens=[1, 1], mode=wl.SCALAR),
    dict(seed=608, ctx=[640, 129], q_lens=[2, 2], mode=wl.NONE),
    # a wide spread of lengths: one long request among short and empty ones
    dict(seed=609, ctx=[40, 9000, 0, 300, 1, 128, 129, 2600], q_lens=[1] * 8),
    dict(seed=610, ctx=[5000, 200, 3100, 64], q_lens=[4, 4, 4, 4]),
    dict(seed=611, ctx=[4100, 90, 700], q_lens=[5, 1, 3], ragged=True),
]


def _max_q_len(w):
    return int(w.q_lens.max()) if w.cu is not None else 0


@pytest.mark.parametrize("kw", CASES, ids=[str(c["seed"]) for c in CASES])
@pytest.mark.parametrize("waves", [0, 4, 8])
def test_balanced_matches_oracle(kw, waves):
    w = wl.small_case(**kw)
    print("balanced case", w.name, "waves", waves, flush=True)
    case = GpuCase(w)
    out = case.decode(partition_mode=BAL, max_q_len=_max_q_len(w), workgroup_waves=waves)
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what=f"{w.name} balanced waves={waves}")


def test_balanced_plan_is_reported():
    w = wl.small_case(seed=612, ctx=[3000, 100], q_lens=[4, 4])
    p = pa.pa_plan_describe(pa.make_config(w.Hkv, w.rows, w.B, w.W, partition_mode=BAL))
    assert p["balanced"] == 1 and p["pages_per_part"] == 0 and p["merge"] == 1


def test_balanced_over_a_bf16_cache():
    w = wl.bf16_kv(wl.small_case(seed=613, ctx=[2200, 70, 900], q_lens=[2, 2, 2]))
    case = GpuCase(w)
    out = case.decode(partition_mode=BAL)
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what="bf16 balanced")


def test_sixty_four_requests():
    """The largest balanced batch: one request per lane of the wave that
    lays out the partitions."""
    rng = np.random.default_rng(614)
    ctx = [int(x) for x in rng.integers(0, 700, size=64)]
    ctx[63] = 2000
    w = wl.small_case(seed=614, ctx=ctx, q_lens=[1] * 64)
    print("64 requests", flush=True)
    case = GpuCase(w)
    out = case.decode(partition_mode=BAL)
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what="64 requests balanced")



def test_one_spare_slot():
    """64 requests over 4 KV heads: 256 / 4 = 64 slots per head is below
    batch + 1, so the call gets 65 slots, one more than the requests.  The
    search for the partition size then spans from ceil(total / 65) up to
    the whole page count."""
    rng = np.random.default_rng(616)
    ctx = [int(x) for x in rng.integers(2, 1500, size=64)]
    ctx[5], ctx[40] = 6000, 4100
    w = wl.small_case(seed=616, ctx=ctx, q_lens=[2] * 64, Hkv=4)
    p = pa.pa_plan_describe(pa.make_config(w.Hkv, w.rows, w.B, w.W, partition_mode=BAL))
    print("one spare slot", p, flush=True)
    case = GpuCase(w)
    out = case.decode(partition_mode=BAL)
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what="64 requests x 4 KV heads balanced")

def test_balanced_and_fixed_agree_and_repeat_bitwise():
    w = wl.small_case(seed=615, ctx=[6000, 130, 2500, 900], q_lens=[4, 4, 4, 4], Hkv=2)
    case = GpuCase(w)
    ref = oracle_out(w)
    outs = [case.decode(out=torch.empty_like(case.out), partition_mode=BAL).clone() for _ in range(3)]
    fixed = case.decode(out=torch.empty_like(case.out), partition_mode=pa.PARTITION_FIXED)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    compare(outs[0], ref, what="balanced")
    compare(fixed, ref, what="fixed")


def test_rows_past_max_q_len_are_zero():
    """A ragged call whose max_q_len understates a request's rows: the rows
    past it have no partials and come out as zeros; the others are exact."""
    w = wl.small_case(seed=616, ctx=[900, 300], q_lens=[4, 2], ragged=True)
    case = GpuCase(w)
    out = case.decode(partition_mode=BAL, max_q_len=2)
    torch.cuda.synchronize()
    ref = oracle_out(w)
    keep = [0, 1, 4, 5]  # rows 0-1 of request 0 and both rows of request 1
    compare(out[keep], np.asarray(ref)[keep], what="rows within max_q_len")
    assert torch.count_nonzero(out[2:4]).item() == 0


def test_balanced_graph_replays_match_eager():
    w = wl.small_case(seed=617, ctx=[3000, 1200, 70], q_lens=[2, 2, 2])
    case = GpuCase(w)
    stream = torch.cuda.Stream()
    # reserve for both plans used below, so no call after the capture grows
    # (and so frees) the scratch the graph holds
    for mode in (BAL, pa.PARTITION_FIXED):
        pa.pa_reserve(pa.make_config(w.Hkv, w.rows, w.B, w.W, partition_mode=mode), stream)
    with torch.cuda.stream(stream):
        eager = case.decode(out=torch.empty_like(case.out), partition_mode=BAL).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(case.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        case.decode(out=out, partition_mode=BAL)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        with torch.cuda.stream(stream):
            other = case.decode(out=torch.empty_like(case.out), partition_mode=pa.PARTITION_FIXED)
        torch.cuda.synchronize()
        compare(other, oracle_out(w), what=f"eager between replays {rep}")
    compare(eager, oracle_out(w), what="eager")


@pytest.mark.parametrize("depth", [3, 4])
def test_balanced_with_deeper_prefetch_rings(depth):
    """The single-row, four-wave variants with three- and four-page rings
    under the balanced layout."""
    for kw in (CASES[0], CASES[1], CASES[8]):
        w = wl.small_case(**kw)
        print("balanced depth", depth, w.name, flush=True)
        case = GpuCase(w)
        out = case.decode(out=torch.empty_like(case.out), partition_mode=BAL, prefetch_depth=depth,
                          workgroup_waves=4)
        torch.cuda.synchronize()
        compare(out, oracle_out(w), what=f"{w.name} balanced depth={depth}")
