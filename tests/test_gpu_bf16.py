"""GPU parity for the unquantized bf16 cache (the control the FP8 cache is
compared against): the writer bit-exact against the oracle's bf16 writer,
and pa_decode over a bf16 cache against the fp64 oracle over the same
cache, element by element on small cases (dense, multi-row, ragged,
sparse; forced partition counts; both workgroup widths) and on sampled
rows of the 128K-context, speculative and sparse shapes at full size."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl
from oracle import writer as owr

from harness import GpuCase, compact_request_oracle, compare, oracle_out

pytestmark = pytest.mark.gpu

FILL = 0x7FC1  # a NaN pattern: any slot the writer should not touch stays NaN


def _bits(t):
    return t.view(torch.int16).cpu().numpy().reshape(-1).view(np.uint16)


@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Hkv", [1, 3])
def test_bf16_writer_bit_exact(in_dtype, Hkv):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(300 + Hkv)
    T, nb = 150, 4
    k = (rng.standard_normal((T, Hkv, 128)) * 4).astype(np.float32)
    v = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    # edge values: ties both ways, signed zero, subnormal, huge, infinities, NaN
    edge = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 1e-40, 3.4e38, np.inf, -np.inf, np.nan,
                     -np.nan, 65504.0, 2 ** -133], np.float32)
    k[0, 0, :len(edge)] = edge
    v[1, Hkv - 1, 100:100 + len(edge)] = edge
    slots = rng.permutation(nb * 128)[:T].astype(np.int64)
    slots[3] = -1
    slots[9] = nb * 128 + 5  # past the cache: skipped
    if in_dtype == torch.bfloat16:
        k, v = wl.bf16_round(k), wl.bf16_round(v)
    print("bf16 writer", in_dtype, Hkv, flush=True)
    kc = torch.full((nb, Hkv, 16384), FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    vc = kc.clone()

    def dev_in(x):
        # bf16 inputs are built from their bits (no conversion by torch,
        # which would canonicalise NaN signs)
        if in_dtype == torch.float32:
            return torch.from_numpy(x).to(dev)
        hi = (x.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
        return torch.from_numpy(hi).to(dev).view(torch.bfloat16)

    pa.kv_quant_write(dev_in(k), dev_in(v), torch.from_numpy(slots).to(dev), kc, vc, None, None,
                      pa.SCALE_NONE)
    torch.cuda.synchronize()
    okc = np.full(nb * Hkv * 16384, FILL, np.uint16)
    ovc = okc.copy()
    owr.write_bf16_ref(k, v, slots, okc, ovc, Hkv)
    assert np.array_equal(_bits(kc), okc), "K bits differ"
    assert np.array_equal(_bits(vc), ovc), "V bits differ"


CASES = [
    dict(seed=401, ctx=[300, 513], q_lens=[1, 1]),                              # two tails
    dict(seed=402, ctx=[1, 2, 127, 128, 129, 1000], q_lens=[1] * 6, Hkv=2),      # page edges
    dict(seed=403, ctx=[700, 45, 300], q_lens=[2, 2, 2]),                        # uniform q_len 2
    dict(seed=404, ctx=[900, 260, 131, 4], q_lens=[4, 4, 4, 4]),                 # uniform q_len 4
    dict(seed=405, ctx=[600, 301, 250, 90], q_lens=[4, 4, 6, 2], ragged=True),   # [4,4,6,2]
    dict(seed=406, ctx=[5000, 3000, 2100], q_lens=[1, 1, 1], Hkv=2, sparse_topk=6),
    dict(seed=407, ctx=[4000, 2500], q_lens=[2, 1], ragged=True, sparse_topk=5),
    dict(seed=408, ctx=[0, 50, 384], q_lens=[1, 1, 1]),                          # empty context
]


@pytest.mark.parametrize("kw", CASES, ids=[str(c["seed"]) for c in CASES])
@pytest.mark.parametrize("parts", [0, 1, 3, 8])
def test_bf16_decode_matches_oracle(kw, parts):
    w = wl.bf16_kv(wl.small_case(**kw))
    print("bf16 decode case", w.name, "parts", parts, flush=True)
    case = GpuCase(w)
    out = case.decode(force_parts=parts) if parts else case.decode()
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what=f"{w.name} parts={parts}")


@pytest.mark.parametrize("kw", [CASES[0], CASES[3], CASES[4], CASES[5]], ids=["401", "404", "405", "406"])
@pytest.mark.parametrize("waves", [4, 8])
def test_bf16_workgroup_widths_match_oracle(kw, waves):
    w = wl.bf16_kv(wl.small_case(**kw))
    case = GpuCase(w)
    ref = oracle_out(w)
    for parts in (0, 1, 5):
        print("bf16 widths", w.name, waves, parts, flush=True)
        out = case.decode(out=torch.empty_like(case.out), force_parts=parts, workgroup_waves=waves)
        torch.cuda.synchronize()
        compare(out, ref, what=f"{w.name} waves={waves} parts={parts}")


def test_bf16_and_fp8_caches_agree_to_fp8_error():
    """The same workload over both caches: outputs differ by no more than
    the e4m3 quantization allows (a loose bound; each side is checked
    exactly against its own oracle above)."""
    w8 = wl.small_case(seed=409, ctx=[2000, 700], q_lens=[1, 1])
    a = GpuCase(w8).decode().float()
    b = GpuCase(wl.bf16_kv(w8)).decode().float()
    torch.cuda.synchronize()
    assert float((a - b).abs().max()) < 0.1
    cos = torch.nn.functional.cosine_similarity(a.reshape(1, -1), b.reshape(1, -1)).item()
    assert cos > 0.995


def _sampled(w, case, sample, what):
    out = case.decode()
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    assert np.all(np.isfinite(g)), what
    for b in sample:
        start = int(w.row_start[b])
        rows = list(range(start, start + int(w.q_lens[b])))
        print(what, "request", b, flush=True)
        compare(g[rows], compact_request_oracle(w, b, rows), what=f"{what} request {b}")
    return out.clone()


def test_bf16_dense_128k():
    w = wl.bf16_kv(wl.c3_dense_128k())
    case = GpuCase(w)
    base = _sampled(w, case, [0, 31], "c3 bf16")
    o = case.decode(out=torch.empty_like(case.out), force_parts=16)
    torch.cuda.synchronize()
    compare(o, base.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what="c3 bf16 parts=16 vs default")
    del case
    torch.cuda.empty_cache()


def test_bf16_spec_uniform_q4():
    w = wl.bf16_kv(wl.c4_spec("uniform"))
    case = GpuCase(w)
    _sampled(w, case, [0, 30], "c4 bf16")


def test_bf16_sparse_tail():
    w = wl.bf16_kv(wl.c5_sparse(True))
    case = GpuCase(w)
    _sampled(w, case, [0, 15], "c5 bf16")
