"""GPU parity of pa_decode_write, one decode step with the cache write done
inside the decode launch.

Each case starts from a cache in which every token of every request is
written by kv_quant_write except the step's own new tokens (the last q_len
positions of each request), whose bytes and scales hold poison.  After
pa_decode_write:
  - the whole cache (codes and scale bits) equals, bit for bit, the cache
    kv_quant_write leaves when it writes every token, and the oracle
    writer's cache;
  - the output matches the fp64 oracle over the fully written cache, to the
    decode tolerance (max|err| <= 1e-2 where |ref| < 4, 2^-7|ref| above,
    cosine >= 0.9999), and the separate writer + decode calls to 4e-3.
The cases cover one-row and two-row workgroups, uniform, odd and ragged
q_len (also with an empty request), new tokens across a page boundary, requests made only of new tokens,
the scalar and no-scale modes, two KV heads, bf16 inputs, forced and
balanced partitions, the in-kernel merge, more new tokens than waves, and
the calls that run unfused (q_len above the fused limit, block-sparse
calls with several rows per request), the bf16 cache (the new tokens
rounded to bf16 and stored in the same launch), and block-sparse single-row calls (partition 0 stores each row's token; the
row attends it only if its page is on the row's list, as after a separate
write), with the new token first in its page and rows whose list leaves
that page out; and the call captured in a graph and replayed over re-poisoned
new-token slots."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl
from oracle import layout as olay

from harness import GpuCase, compare, oracle_cache, oracle_out, poison_arrays
from oracle import writer as owr

pytestmark = pytest.mark.gpu

CASES = [
    dict(seed=401, ctx=[300, 513], q_lens=[1, 1]),                              # one-row, two tails
    dict(seed=402, ctx=[700, 1300, 256], q_lens=[4, 4, 4]),                     # two-row, uniform q_len 4
    dict(seed=403, ctx=[260, 129], q_lens=[3, 3]),                              # odd q_len; new tokens cross a page
    dict(seed=404, ctx=[800, 500, 300, 90], q_lens=[4, 1, 6, 2], ragged=True),  # ragged
    dict(seed=405, ctx=[4, 1, 2], q_lens=[4, 1, 2], ragged=True),               # only new tokens
    dict(seed=406, ctx=[1500, 800], q_lens=[1, 1], mode=wl.SCALAR),
    dict(seed=407, ctx=[640, 129], q_lens=[2, 2], mode=wl.NONE),
    dict(seed=408, ctx=[400, 131], q_lens=[2, 2], Hkv=2),
    dict(seed=409, ctx=[600, 2000], q_lens=[16, 16]),                           # more new tokens than waves
    dict(seed=440, ctx=[300, 50, 513], q_lens=[1, 0, 1], ragged=True),          # one-row, an empty request
    dict(seed=441, ctx=[700, 90, 260], q_lens=[2, 0, 3], ragged=True),          # two-row, an empty request
]


def _new_token_poison(case, w, slots):
    """Poison the new tokens' codes and scales in the GPU cache (they are
    written by the call under test)."""
    kc = case.kc.view(torch.uint8).view(-1)
    vc = case.vc.view(torch.uint8).view(-1)
    kidx, vidx, sidx = [], [], []
    d = np.arange(128)
    for s in slots:
        page, o = divmod(int(s), 128)
        for h in range(w.Hkv):
            base = (page * w.Hkv + h) * 16384
            kidx.append(base + olay.k_offset(o, d))
            vidx.append(base + olay.v_offset(o, d))
            sidx.append((page * w.Hkv + h) * 128 + o)
    dev = kc.device
    kidx = torch.from_numpy(np.concatenate(kidx).astype(np.int64)).to(dev)
    vidx = torch.from_numpy(np.concatenate(vidx).astype(np.int64)).to(dev)
    kc[kidx] = 0x5A
    vc[vidx] = 0x3C
    if w.mode == wl.PER_TOKEN:
        sidx = torch.from_numpy(np.asarray(sidx, np.int64)).to(dev)
        case.ks.view(-1)[sidx] = 1e3
        case.vs.view(-1)[sidx] = 1e3


def _oracle_cache_bf16_inputs(w):
    """The oracle writer's cache when the K/V inputs are bf16 (each value
    rounded to bf16 before quantization, as the GPU call receives them)."""
    kc, vc, ks, vs = poison_arrays(w)
    ks_in = np.array([w.k_scalar], np.float32)
    vs_in = np.array([w.v_scalar], np.float32)
    for b in range(w.B):
        k, v, s = w.request_kv(b)
        k, v = wl.bf16_round(k), wl.bf16_round(v)
        if w.mode == wl.SCALAR:
            owr.quant_write_ref(k, v, s, kc, vc, ks_in, vs_in, w.mode, w.Hkv)
        else:
            owr.quant_write_ref(k, v, s, kc, vc, ks, vs, w.mode, w.Hkv)
    ksa, vsa = (ks_in, vs_in) if w.mode == wl.SCALAR else ((None, None) if w.mode == wl.NONE else (ks, vs))
    return kc, vc, ks, vs, ksa, vsa


def _snapshot(case):
    snap = [case.kc.view(torch.uint8).clone(), case.vc.view(torch.uint8).clone()]
    if case.ks is not None:
        snap += [case.ks.view(torch.int32).clone(), case.vs.view(torch.int32).clone()]
    return snap


def _run(case, w, k, v, slots, out, **kw):
    mq = int(w.q_lens.max()) if w.cu is not None else 0
    pa.pa_decode_write(case.q, k, v, slots, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt, case.ctx,
                       case.cu, case.mode, out, max_q_len=mq, sparse_page_idx=case.sp, **kw)
    return out


def _check_step(w, in_dtype=torch.float32, what="", runs=({},)):
    case = GpuCase(w, in_dtype=in_dtype)
    full = _snapshot(case)  # every token written by kv_quant_write
    ref_sep = case.decode(out=torch.empty_like(case.out),
                          max_q_len=int(w.q_lens.max()) if w.cu is not None else 0)
    torch.cuda.synchronize()
    ocache = _oracle_cache_bf16_inputs(w) if in_dtype == torch.bfloat16 else oracle_cache(w)
    ref64 = oracle_out(w, cache=ocache)
    k, v, s = w.step_tokens()
    kt = torch.from_numpy(k).to(case.dev).to(in_dtype)
    vt = torch.from_numpy(v).to(case.dev).to(in_dtype)
    st = torch.from_numpy(s).to(case.dev)
    for kw in runs:
        tag = f"{what} {kw}"
        print("fused write case", w.name, tag, flush=True)
        _new_token_poison(case, w, s)
        torch.cuda.synchronize()
        out = _run(case, w, kt, vt, st, torch.empty_like(case.out), **kw)
        torch.cuda.synchronize()
        after = _snapshot(case)
        for a, b, name in zip(after, full, ("k codes", "v codes", "k scales", "v scales")):
            assert torch.equal(a, b), f"{tag}: {name} differ from kv_quant_write's"
        # and from the oracle writer's (codes and scale bits)
        assert np.array_equal(after[0].cpu().numpy().reshape(-1), ocache[0].reshape(-1)), f"{tag}: K vs oracle"
        assert np.array_equal(after[1].cpu().numpy().reshape(-1), ocache[1].reshape(-1)), f"{tag}: V vs oracle"
        if w.mode == wl.PER_TOKEN:
            assert np.array_equal(after[2].cpu().numpy().reshape(-1), ocache[2].view(np.int32).reshape(-1))
            assert np.array_equal(after[3].cpu().numpy().reshape(-1), ocache[3].view(np.int32).reshape(-1))
        compare(out, ref64, what=f"{tag} vs oracle")
        compare(out, ref_sep.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{tag} vs separate calls")


@pytest.mark.parametrize("kw", CASES, ids=[str(c["seed"]) for c in CASES])
def test_fused_write_step(kw):
    w = wl.small_case(**kw)
    runs = [{}, dict(force_parts=1), dict(force_parts=3), dict(force_parts=8),
            dict(partition_mode=pa.PARTITION_BALANCED), dict(merge_mode=pa.MERGE_IN_KERNEL, force_parts=3)]
    _check_step(w, runs=runs, what=w.name)


def test_fused_write_bf16_inputs_and_widths():
    w = wl.small_case(seed=410, ctx=[900, 333, 128], q_lens=[2, 2, 2])
    _check_step(w, in_dtype=torch.bfloat16, what="bf16 inputs",
                runs=({}, dict(workgroup_waves=4), dict(workgroup_waves=8), dict(force_parts=5)))


def test_unfused_fallbacks():
    # q_len above the fused limit, and a forced deeper ring: writer + decode
    w = wl.small_case(seed=411, ctx=[700, 300], q_lens=[17, 17])
    _check_step(w, what="q_len 17", runs=({}, dict(force_parts=2)))
    w = wl.small_case(seed=412, ctx=[700, 300], q_lens=[1, 1])
    _check_step(w, what="depth 3", runs=(dict(prefetch_depth=3),))
    # block-sparse calls with more than one row per request
    w = wl.small_case(seed=415, ctx=[2000, 900], q_lens=[2, 2], sparse_topk=4)
    _check_step(w, what="sparse q_len 2", runs=({}, dict(force_parts=2)))
    w = wl.small_case(seed=416, ctx=[1500, 600, 300], q_lens=[3, 1, 2], ragged=True, sparse_topk=3)
    _check_step(w, what="sparse ragged", runs=({},))


BF16_CASES = [
    dict(seed=413, ctx=[500, 260], q_lens=[2, 2]),                              # two-row (four waves)
    dict(seed=417, ctx=[300, 513], q_lens=[1, 1]),                              # one-row, two tails
    dict(seed=418, ctx=[800, 500, 300, 90], q_lens=[4, 1, 6, 2], ragged=True),  # ragged
    dict(seed=419, ctx=[600, 2000], q_lens=[16, 16]),                           # more new tokens than waves
    dict(seed=420, ctx=[400, 131], q_lens=[3, 3], Hkv=2),                       # new tokens cross a page
    dict(seed=421, ctx=[700, 1300, 513], q_lens=[1, 1, 1], sparse_topk=3),      # block-sparse
]


def _bf16_slots_elements(kc16, vc16, w, slots):
    """The K and V elements of the new tokens' slots (every head, every dim)."""
    d = np.arange(128)
    ki, vi = [], []
    for s1 in slots:
        page, o = divmod(int(s1), 128)
        for h in range(w.Hkv):
            base = (page * w.Hkv + h) * 16384
            ki.append(base + olay.k_offset_bf16(o, d))
            vi.append(base + olay.v_offset_bf16(o, d))
    ki, vi = np.concatenate(ki), np.concatenate(vi)
    return kc16[ki], vc16[vi], ki, vi


@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("kw", BF16_CASES, ids=[str(c["seed"]) for c in BF16_CASES])
def test_fused_write_bf16_cache(kw, in_dtype):
    """The unquantized cache: the new tokens are rounded to bf16 and stored
    inside the decode launch, bit-equal to kv_quant_write's and the oracle
    writer's elements."""
    w = wl.bf16_kv(wl.small_case(**kw))
    case = GpuCase(w, in_dtype=in_dtype)
    mq = int(w.q_lens.max()) if w.cu is not None else 0
    ref_sep = case.decode(out=torch.empty_like(case.out), max_q_len=mq)
    torch.cuda.synchronize()
    full = [case.kc.view(torch.int16).clone(), case.vc.view(torch.int16).clone()]
    okc, ovc = oracle_cache(w)[:2]
    ref64 = oracle_out(w)
    k, v, s = w.step_tokens()
    kt = torch.from_numpy(k).to(case.dev).to(in_dtype)
    vt = torch.from_numpy(v).to(case.dev).to(in_dtype)
    st = torch.from_numpy(s).to(case.dev)
    ok_new, ov_new, ki, vi = _bf16_slots_elements(okc, ovc, w, s)
    kit = torch.from_numpy(ki.astype(np.int64)).to(case.dev)
    vit = torch.from_numpy(vi.astype(np.int64)).to(case.dev)
    runs = [{}, dict(force_parts=1), dict(force_parts=3)]
    if int(w.q_lens.max()) == 1 and w.sparse is None:
        runs.append(dict(workgroup_waves=8))
    for kwr in runs:
        tag = f"{w.name} bf16 cache, {in_dtype} inputs, {kwr}"
        print("fused write case", tag, flush=True)
        # overwrite the new tokens' elements with a pattern; the call writes them back
        case.kc.view(torch.int16).view(-1)[kit] = 0x1234
        case.vc.view(torch.int16).view(-1)[vit] = 0x1234
        torch.cuda.synchronize()
        out = _run(case, w, kt, vt, st, torch.empty_like(case.out), **kwr)
        torch.cuda.synchronize()
        assert torch.equal(case.kc.view(torch.int16), full[0]), f"{tag}: K differs from kv_quant_write's"
        assert torch.equal(case.vc.view(torch.int16), full[1]), f"{tag}: V differs from kv_quant_write's"
        g = case.kc.view(torch.int16).view(-1)[kit].cpu().numpy().view(np.uint16)
        assert np.array_equal(g, ok_new), f"{tag}: new K elements vs the oracle writer"
        g = case.vc.view(torch.int16).view(-1)[vit].cpu().numpy().view(np.uint16)
        assert np.array_equal(g, ov_new), f"{tag}: new V elements vs the oracle writer"
        compare(out, ref64, what=f"{tag} vs oracle")
        compare(out, ref_sep.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{tag} vs separate calls")


def test_fused_write_refuses_before_launch():
    w = wl.small_case(seed=414, ctx=[300], q_lens=[2])
    case = GpuCase(w)
    k, v, s = w.step_tokens()
    kt = torch.from_numpy(k[:1]).to(case.dev)
    vt = torch.from_numpy(v[:1]).to(case.dev)
    st = torch.from_numpy(s[:1]).to(case.dev)
    before = _snapshot(case)
    with pytest.raises(RuntimeError, match="query rows"):
        _run(case, w, kt, vt, st, torch.empty_like(case.out))
    torch.cuda.synchronize()
    for a, b in zip(_snapshot(case), before):
        assert torch.equal(a, b)


SPARSE_CASES = [
    dict(seed=431, ctx=[700, 1300, 513], q_lens=[1, 1, 1], sparse_topk=3),             # 513: first token of page 4
    dict(seed=432, ctx=[2000, 129], q_lens=[1, 1], sparse_topk=2, mode=wl.SCALAR),     # 129: first token of page 1
    dict(seed=433, ctx=[1025, 400], q_lens=[1, 1], sparse_topk=4, mode=wl.NONE, Hkv=2),
]


@pytest.mark.parametrize("drop", [False, True], ids=["listed", "unlisted"])
@pytest.mark.parametrize("kw", SPARSE_CASES, ids=[str(c["seed"]) for c in SPARSE_CASES])
def test_fused_write_sparse(kw, drop):
    w = wl.small_case(**kw)
    case = GpuCase(w)
    full = _snapshot(case)
    if drop:
        # odd rows no longer list the page that holds their new token
        sp = w.sparse.copy()
        for r in range(1, w.rows, 2):
            last = (int(w.ctx[r]) - 1) // 128
            sp[r][sp[r] == last] = -1
        w.sparse = sp
        case.sp = torch.from_numpy(sp).to(case.dev)
    ocache = oracle_cache(w)
    ref64 = oracle_out(w, cache=ocache)
    ref_sep = case.decode(out=torch.empty_like(case.out))
    torch.cuda.synchronize()
    k, v, s = w.step_tokens()
    kt = torch.from_numpy(k).to(case.dev)
    vt = torch.from_numpy(v).to(case.dev)
    st = torch.from_numpy(s).to(case.dev)
    for kwr in ({}, dict(force_parts=1), dict(force_parts=2), dict(force_parts=3)):
        tag = f"{w.name} {'unlisted' if drop else 'listed'} {kwr}"
        print("fused write sparse case", tag, flush=True)
        _new_token_poison(case, w, s)
        torch.cuda.synchronize()
        out = torch.empty_like(case.out)
        pa.pa_decode_write(case.q, kt, vt, st, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt, case.ctx,
                           None, case.mode, out, sparse_page_idx=case.sp, **kwr)
        torch.cuda.synchronize()
        after = _snapshot(case)
        for a, b, name in zip(after, full, ("k codes", "v codes", "k scales", "v scales")):
            assert torch.equal(a, b), f"{tag}: {name} differ from kv_quant_write's"
        assert np.array_equal(after[0].cpu().numpy().reshape(-1), ocache[0].reshape(-1)), f"{tag}: K vs oracle"
        assert np.array_equal(after[1].cpu().numpy().reshape(-1), ocache[1].reshape(-1)), f"{tag}: V vs oracle"
        compare(out, ref64, what=f"{tag} vs oracle")
        compare(out, ref_sep.float().cpu().numpy(), atol=4e-3, cos_min=0.99999, what=f"{tag} vs separate calls")


GRAPH_CASES = [
    dict(seed=450, ctx=[1300, 700, 513], q_lens=[1, 1, 1]),                      # one-row: write before the stream
    dict(seed=451, ctx=[900, 260], q_lens=[4, 4]),                               # two-row: write after the stream
    dict(seed=452, ctx=[2000, 1300], q_lens=[1, 1], sparse_topk=4),              # block-sparse
    dict(seed=453, ctx=[800, 333], q_lens=[1, 1], bf16=True),                    # bf16 cache
]


@pytest.mark.parametrize("kw", GRAPH_CASES, ids=[str(c["seed"]) for c in GRAPH_CASES])
def test_fused_write_graph_replay(kw):
    """pa_decode_write captured in a graph (scratch reserved first) and
    replayed several times over a cache whose new-token slots are poisoned
    again before each replay, with eager calls between the replays: every
    replay leaves the cache kv_quant_write leaves and the eager output, bit
    for bit."""
    kw = dict(kw)
    bf = kw.pop("bf16", False)
    w = wl.small_case(**kw)
    if bf:
        w = wl.bf16_kv(w)
    case = GpuCase(w)
    k, v, s = w.step_tokens()
    kt = torch.from_numpy(k).to(case.dev)
    vt = torch.from_numpy(v).to(case.dev)
    st = torch.from_numpy(s).to(case.dev)
    if bf:
        full = [case.kc.view(torch.int16).clone(), case.vc.view(torch.int16).clone()]
        _, _, ki, vi = _bf16_slots_elements(np.zeros(case.kc.numel(), np.uint16),
                                            np.zeros(case.vc.numel(), np.uint16), w, s)
        kit = torch.from_numpy(ki.astype(np.int64)).to(case.dev)
        vit = torch.from_numpy(vi.astype(np.int64)).to(case.dev)

        def poison():
            case.kc.view(torch.int16).view(-1)[kit] = 0x1234
            case.vc.view(torch.int16).view(-1)[vit] = 0x1234

        def cache_ok():
            return torch.equal(case.kc.view(torch.int16), full[0]) and torch.equal(case.vc.view(torch.int16), full[1])
    else:
        full = _snapshot(case)

        def poison():
            _new_token_poison(case, w, s)

        def cache_ok():
            return all(torch.equal(a, b) for a, b in zip(_snapshot(case), full))
    stream = torch.cuda.Stream()
    cfg = pa.make_config(w.Hkv, w.rows, w.B, w.W, topk=0 if w.sparse is None else w.sparse.shape[1],
                         scale_mode=w.mode, kv_dtype=3 if bf else 1)
    pa.pa_reserve(cfg, stream)
    print("fused write graph case", w.name, pa.pa_plan_describe(cfg)["rows_per_group"], flush=True)
    poison()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        eager = _run(case, w, kt, vt, st, torch.empty_like(case.out)).clone()
    torch.cuda.synchronize()
    assert cache_ok(), "eager call: cache differs from kv_quant_write's"
    compare(eager, oracle_out(w), what=f"{w.name} eager")
    out = torch.empty_like(case.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        _run(case, w, kt, vt, st, out)
    for rep in range(3):
        poison()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert cache_ok(), f"replay {rep}: cache differs from kv_quant_write's"
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}: output"
        with torch.cuda.stream(stream):
            other = case.decode(out=torch.empty_like(case.out))
        torch.cuda.synchronize()
        compare(other, oracle_out(w), what=f"{w.name} eager decode between replays {rep}")
