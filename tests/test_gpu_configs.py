"""The five workloads at full size, in the launch configuration the bench
times: the cache is written by kv_quant_write, and the sampled requests'
pages are compared with the oracle writer's byte for byte (codes and scale
bits); sampled rows are checked
element by element against the oracle (rebuilt on a compact cache of just
those requests' pages); every row is checked against properties that hold
at any size (finite, the default plan agrees with forced partition counts
and with the other partition mode)."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, assert_request_bytes, compact_request_cache, compact_request_oracle, compare

pytestmark = pytest.mark.gpu


def _check(w, case, sample_requests, what):
    out = case.decode()
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g)), what
    for b in sample_requests:
        start = int(w.row_start[b])
        rows = list(range(start, start + int(w.q_lens[b])))
        print(what, "request", b, "rows", rows, flush=True)
        cc = compact_request_cache(w, b)
        # the cache kv_quant_write wrote for this request: every byte and scale
        assert_request_bytes(w, b, case, cc)
        ref = compact_request_oracle(w, b, rows, cc)
        compare(g[rows], ref, what=f"{what} request {b}")
    return out.clone()


def _parts_agree(case, base, parts_list, what):
    for p in parts_list:
        o = case.decode(out=torch.empty_like(case.out), force_parts=p)
        torch.cuda.synchronize()
        compare(o, base.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{what} parts={p} vs default")


def _modes_agree(w, case, base, what):
    """Fixed and length-balanced partitions against the default plan (the
    ragged calls with max_q_len, which balanced partitions need)."""
    mq = int(w.q_lens.max()) if w.cu is not None else 0
    for mode in (pa.PARTITION_FIXED, pa.PARTITION_BALANCED):
        o = case.decode(out=torch.empty_like(case.out), partition_mode=mode, max_q_len=mq)
        torch.cuda.synchronize()
        compare(o, base.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{what} mode={mode} vs default")


def test_c1_tiny():
    w = wl.c1_tiny()
    case = GpuCase(w)
    _check(w, case, [0, 1], "c1")


def test_c2_dense_8k():
    w = wl.c2_dense_8k()
    case = GpuCase(w)
    base = _check(w, case, range(4), "c2")
    _parts_agree(case, base, [1, 8, 32], "c2")
    _modes_agree(w, case, base, "c2")


@pytest.mark.parametrize("mode", [wl.PER_TOKEN, wl.SCALAR])
def test_c3_dense_128k(mode):
    w = wl.c3_dense_128k(mode)
    case = GpuCase(w)
    base = _check(w, case, [0, 17, 31], f"c3 mode={mode}")
    _parts_agree(case, base, [8, 16, 32], f"c3 mode={mode}")
    _modes_agree(w, case, base, f"c3 mode={mode}")
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["uniform", "uniform_cu", "ragged", "mixed"])
def test_c4_spec(kind):
    w = wl.c4_spec(kind)
    case = GpuCase(w)
    short = [b for b in range(w.B) if w.q_lens[b] != w.q_lens.max()]
    sample = sorted(set([0, w.B - 1] + short[:2]))
    base = _check(w, case, sample, f"c4 {kind}")
    _parts_agree(case, base, [4, 16], f"c4 {kind}")
    _modes_agree(w, case, base, f"c4 {kind}")


@pytest.mark.parametrize("tail", [False, True])
def test_c5_sparse(tail):
    w = wl.c5_sparse(tail)
    case = GpuCase(w)
    base = _check(w, case, [0, 7, 15], f"c5 tail={tail}")
    _parts_agree(case, base, [1, 4, 32], f"c5 tail={tail}")
