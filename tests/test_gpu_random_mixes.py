"""GPU parity of pa_decode against the fp64 oracle over seeded random call
mixes: batch size, KV heads, scale mode, uniform / ragged / block-sparse
rows, context lengths drawn around page edges, and the plan options
(partition mode, forced partition counts, workgroup width, prefetch depth,
merge placement, the max_q_len hint), each drawn only where the option is
served.  Every output element is held to max|err| <= 1e-2 and cosine >=
0.9999, the tolerance stated for this path.  Every draw (and every fourth
over a bf16 cache) also runs as one pa_decode_write step from a cache whose
new-token slots hold poison: the cache afterwards equals kv_quant_write's
bit for bit."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl

from harness import GpuCase, compare, oracle_out

SEEDS = list(range(601, 665))


def draw(seed):
    """One call: the workload arguments and the pa_decode_ex options."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    Hkv = int(rng.choice([1, 1, 2]))
    mode = [wl.PER_TOKEN, wl.PER_TOKEN, wl.PER_TOKEN, wl.SCALAR, wl.NONE][int(rng.integers(0, 5))]
    kind = ["uniform", "ragged", "sparse"][int(rng.integers(0, 3))]
    if kind == "uniform":
        q_lens = [int(rng.integers(1, 6))] * B
    elif kind == "ragged":
        q_lens = [int(x) for x in rng.integers(1, 8, size=B)]
    else:
        q_lens = [int(x) for x in rng.integers(1, 3, size=B)]
    topk = int(rng.integers(1, 7)) if kind == "sparse" else 0
    ctx = []
    for L in q_lens:
        lo = max(L, 128 * topk)
        if rng.random() < 0.5:
            # next to a page edge: k*128 - 1, k*128 or k*128 + 1 tokens
            c = 128 * int(rng.integers(1, 20)) + int(rng.integers(-1, 2))
        else:
            c = int(rng.integers(1, 2600))
        ctx.append(max(c, lo))
    w = wl.small_case(seed=seed, ctx=ctx, q_lens=q_lens, Hkv=Hkv, ragged=kind != "uniform", mode=mode,
                      sparse_topk=topk)

    opts = {}
    hint = kind != "uniform" and rng.random() < 0.6
    if hint:
        opts["max_q_len"] = max(q_lens)
    dense = kind != "sparse"
    balanced_ok = dense and (kind == "uniform" or hint)
    pm = int(rng.choice([0, 1, 2] if balanced_ok else [0, 1]))
    opts["partition_mode"] = pm
    if pm == 1 and rng.random() < 0.5:
        opts["force_parts"] = int(rng.choice([1, 2, 5, 13]))
    if pm == 1 and rng.random() < 0.3:
        opts["merge_mode"] = pa.MERGE_IN_KERNEL
    waves = int(rng.choice([0, 4, 8]))
    if waves:
        opts["workgroup_waves"] = waves
    if dense and waves != 8 and rng.random() < 0.3:
        opts["prefetch_depth"] = int(rng.choice([3, 4]))
    return w, opts


@pytest.mark.gpu
@pytest.mark.parametrize("seed", SEEDS)
def test_random_call_matches_oracle(seed):
    w, opts = draw(seed)
    print("random mix", seed, "B", w.B, "Hkv", w.Hkv, "mode", w.mode, "q_lens", list(w.q_lens), "ctx",
          list(w.ctx), "topk", 0 if w.sparse is None else w.sparse.shape[1], "opts", opts, flush=True)
    case = GpuCase(w)
    out = case.decode(**opts)
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what=f"random mix {seed} {opts}")



@pytest.mark.gpu
@pytest.mark.parametrize("seed", SEEDS[::4])
def test_random_call_over_a_bf16_cache_matches_oracle(seed):
    """The same draws over an unquantized bf16 cache (no scales)."""
    w, opts = draw(seed)
    w = wl.bf16_kv(w)
    print("random mix bf16", seed, "q_lens", list(w.q_lens), "ctx", list(w.ctx), "opts", opts, flush=True)
    out = GpuCase(w).decode(**opts)
    torch.cuda.synchronize()
    compare(out, oracle_out(w), what=f"random mix bf16 {seed} {opts}")

def _write_step(w, opts, seed):
    """One decode step through pa_decode_write from a cache whose new-token
    slots hold poison: the cache after the call equals kv_quant_write's bit
    for bit, and the output matches the oracle."""
    from test_gpu_fused_write import _bf16_slots_elements, _new_token_poison, _snapshot

    case = GpuCase(w)
    k, v, s = w.step_tokens()
    kt, vt, st = (torch.from_numpy(x).to(case.dev) for x in (k, v, s))
    # the reference cache: every step token written by kv_quant_write too (a
    # block-sparse workload writes only the pages its lists name, and a
    # request's earlier new tokens can sit on a page before the listed last one)
    pa.kv_quant_write(kt, vt, st, case.kc, case.vc, case.ks_arg, case.vs_arg, case.mode)
    torch.cuda.synchronize()
    if w.kv_dtype == "bf16":
        full = [case.kc.view(torch.int16).clone(), case.vc.view(torch.int16).clone()]
        _, _, ki, vi = _bf16_slots_elements(np.zeros(case.kc.numel(), np.uint16),
                                            np.zeros(case.vc.numel(), np.uint16), w, s)
        case.kc.view(torch.int16).view(-1)[torch.from_numpy(ki.astype(np.int64)).to(case.dev)] = 0x1234
        case.vc.view(torch.int16).view(-1)[torch.from_numpy(vi.astype(np.int64)).to(case.dev)] = 0x1234
        snap = lambda: [case.kc.view(torch.int16), case.vc.view(torch.int16)]
    else:
        full = _snapshot(case)
        _new_token_poison(case, w, s)
        snap = lambda: _snapshot(case)
    out = torch.empty_like(case.out)
    pa.pa_decode_write(case.q, kt, vt, st, case.kc, case.vc, case.ks_arg, case.vs_arg, case.bt,
                       case.ctx, case.cu, case.mode, out, sparse_page_idx=case.sp, **opts)
    torch.cuda.synchronize()
    for a, b in zip(snap(), full):
        assert torch.equal(a, b), f"random step {seed}: cache differs from kv_quant_write's"
    compare(out, oracle_out(w), what=f"random step {seed} {opts}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", SEEDS)
def test_random_step_with_the_write_inside_the_decode(seed):
    """Every draw as one decode step through pa_decode_write.  Draws with a
    forced deeper ring, (ragged) no max_q_len hint, more than 16 rows per
    request or several rows per block-sparse request run the writer and the
    decode separately inside the call; the rest write inside the decode."""
    w, opts = draw(seed)
    print("random step", seed, "B", w.B, "Hkv", w.Hkv, "mode", w.mode, "q_lens", list(w.q_lens), "ctx",
          list(w.ctx), "sparse", w.sparse is not None, "opts", opts, flush=True)
    _write_step(w, opts, seed)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", SEEDS[::4])
def test_random_step_over_a_bf16_cache(seed):
    w, opts = draw(seed)
    w = wl.bf16_kv(w)
    print("random bf16 step", seed, "q_lens", list(w.q_lens), "sparse", w.sparse is not None, "opts", opts,
          flush=True)
    _write_step(w, opts, seed)


def test_draws_cover_every_kind_and_option():
    """The seeds above reach every call kind, scale mode and plan option."""
    kinds, modes, keys, pms = set(), set(), set(), set()
    for s in SEEDS:
        w, opts = draw(s)
        kinds.add("sparse" if w.sparse is not None else ("ragged" if w.cu is not None else "uniform"))
        modes.add(w.mode)
        keys |= set(opts)
        pms.add(opts["partition_mode"])
    assert kinds == {"uniform", "ragged", "sparse"}
    assert modes == {wl.PER_TOKEN, wl.SCALAR, wl.NONE}
    assert pms == {0, 1, 2}
    assert {"max_q_len", "force_parts", "merge_mode", "workgroup_waves", "prefetch_depth"} <= keys
