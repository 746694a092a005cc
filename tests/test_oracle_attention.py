"""Pins for the oracle's attention against things other than itself:
a loop-only brute force with exactly rounded sums on tiny inputs, closed
forms (constant V, one-token context, zero query), the identities the
method relies on (block-table permutation, scalar fold, split-K merge,
multi-row = single-row at the shifted cutoff, sparse over all pages =
dense), and torch's fp64 scaled_dot_product_attention for GQA = MHA with
K/V repeated 16 times."""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as att
from oracle import e4m3, layout, writer

PT, SC, NO = att.PER_TOKEN, att.SCALAR, att.NONE


def build_cache(w, poison=True):
    """Oracle-side cache for a workload: poison everywhere, then the written
    pages through the reference writer."""
    nb, Hkv = w.num_blocks, w.Hkv
    rng = np.random.default_rng(w.seed + 99)
    if poison:
        kc = rng.integers(0, 0x7F, size=nb * Hkv * 16384).astype(np.uint8)
        vc = rng.integers(0, 0x7F, size=nb * Hkv * 16384).astype(np.uint8)
    else:
        kc = np.zeros(nb * Hkv * 16384, np.uint8)
        vc = kc.copy()
    ks = np.full(nb * Hkv * 128, 1e3, dtype=np.float32)
    vs = ks.copy()
    if w.mode == SC:
        ks_in = np.array([w.k_scalar], np.float32)
        vs_in = np.array([w.v_scalar], np.float32)
    for b in range(w.B):
        k, v, s = w.request_kv(b)
        if w.mode == SC:
            writer.quant_write_ref(k, v, s, kc, vc, ks_in, vs_in, SC, Hkv)
        else:
            writer.quant_write_ref(k, v, s, kc, vc, ks, vs, w.mode, Hkv)
    if w.mode == SC:
        return kc, vc, ks_in, vs_in
    if w.mode == NO:
        return kc, vc, None, None
    return kc, vc, ks, vs


def run_ref(w, cache, **kw):
    kc, vc, ks, vs = cache
    return att.attention_ref(w.q, kc, vc, ks, vs, w.block_table, w.ctx, w.cu, w.sparse,
                             w.mode, w.Hkv, **kw)


TINY = [
    dict(seed=11, ctx=[1, 5, 130], q_lens=[1, 1, 1], Hkv=1),
    dict(seed=12, ctx=[7, 140], q_lens=[2, 2], Hkv=2),
    dict(seed=13, ctx=[9, 3, 131], q_lens=[3, 1, 2], Hkv=1, ragged=True),
    dict(seed=14, ctx=[129, 200], q_lens=[1, 1], Hkv=1, mode=SC),
    dict(seed=15, ctx=[60, 257], q_lens=[1, 2], Hkv=1, mode=NO, ragged=True),
]


@pytest.mark.parametrize("cfg", TINY)
def test_matches_bruteforce(cfg):
    w = wl.small_case(**cfg)
    cache = build_cache(w)
    kc, vc, ks, vs = cache
    ref = run_ref(w, cache)
    bf = att.attention_bruteforce(w.q, kc, vc, ks, vs, w.block_table, w.ctx, w.cu, w.sparse,
                                  w.mode, w.Hkv)
    np.testing.assert_allclose(ref, bf, rtol=1e-12, atol=1e-13)


def test_sparse_matches_bruteforce():
    w = wl.small_case(seed=16, ctx=[600, 777], q_lens=[1, 2], ragged=True, sparse_topk=3)
    w.sparse[1, 0] = -1  # a padding entry
    cache = build_cache(w)
    kc, vc, ks, vs = cache
    ref = run_ref(w, cache)
    bf = att.attention_bruteforce(w.q, kc, vc, ks, vs, w.block_table, w.ctx, w.cu, w.sparse,
                                  w.mode, w.Hkv)
    np.testing.assert_allclose(ref, bf, rtol=1e-12, atol=1e-13)


def test_constant_v_returns_v():
    w = wl.small_case(seed=21, ctx=[300, 45], q_lens=[1, 1], mode=NO)
    kc, vc, ks, vs = build_cache(w)
    # overwrite every V code with one value: 0x3C = 1.5
    vc[:] = 0x3C
    out = att.attention_ref(w.q, kc, vc, None, None, w.block_table, w.ctx, None, None, NO, 1)
    np.testing.assert_allclose(out, 1.5, rtol=0, atol=1e-14)


def test_one_token_context_returns_scaled_v():
    w = wl.small_case(seed=22, ctx=[1, 1], q_lens=[1, 1])
    kc, vc, ks, vs = build_cache(w)
    out = run_ref(w, (kc, vc, ks, vs))
    for b in range(2):
        P = int(w.block_table[b, 0])
        codes = vc[int(layout.block_base(P, 0, 1)) + layout.v_offset(0, np.arange(128))]
        want = e4m3.decode(codes) * float(vs[layout.scale_index(P, 0, 0, 1)])
        for j in range(16):
            np.testing.assert_allclose(out[b, j], want, rtol=1e-15, atol=0)


def test_zero_query_gives_mean_of_v():
    w = wl.small_case(seed=23, ctx=[77, 300], q_lens=[1, 1])
    w.q[:] = 0
    kc, vc, ks, vs = build_cache(w)
    out = run_ref(w, (kc, vc, ks, vs))
    for b in range(2):
        vals = []
        for t in range(int(w.ctx[b])):
            P = int(w.block_table[b, t // 128])
            o = t % 128
            codes = vc[int(layout.block_base(P, 0, 1)) + layout.v_offset(o, np.arange(128))]
            vals.append(e4m3.decode(codes) * float(vs[layout.scale_index(P, 0, o, 1)]))
        np.testing.assert_allclose(out[b, 0], np.mean(vals, axis=0), rtol=1e-12, atol=1e-14)


def test_block_table_permutation_is_bitwise_invariant():
    w = wl.small_case(seed=24, ctx=[400, 260], q_lens=[1, 1], Hkv=2)
    kc, vc, ks, vs = build_cache(w)
    out = run_ref(w, (kc, vc, ks, vs))
    # move every physical page to a new id (copy bytes and scales), rebuild table
    nb = w.num_blocks
    perm = np.random.default_rng(5).permutation(nb)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    ks2, vs2 = np.empty_like(ks), np.empty_like(vs)
    for P in range(nb):
        Q = int(perm[P])
        for h in range(2):
            a, bq = int(layout.block_base(P, h, 2)), int(layout.block_base(Q, h, 2))
            kc2[bq:bq + 16384] = kc[a:a + 16384]
            vc2[bq:bq + 16384] = vc[a:a + 16384]
            sa, sb = (P * 2 + h) * 128, (Q * 2 + h) * 128
            ks2[sb:sb + 128] = ks[sa:sa + 128]
            vs2[sb:sb + 128] = vs[sa:sa + 128]
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    out2 = att.attention_ref(w.q, kc2, vc2, ks2, vs2, bt2, w.ctx, None, None, PT, 2)
    assert np.array_equal(out, out2)


def test_scalar_fold_equals_unfolded():
    w = wl.small_case(seed=25, ctx=[333, 129, 5], q_lens=[1, 1, 1], mode=SC)
    kc, vc, ks, vs = build_cache(w)
    plain = run_ref(w, (kc, vc, ks, vs))
    folded = att.attention_ref_scalar_folded(w.q, kc, vc, ks, vs, w.block_table, w.ctx)
    np.testing.assert_allclose(plain, folded, rtol=1e-12, atol=1e-15)


def test_per_token_equal_scales_equals_scalar():
    w = wl.small_case(seed=26, ctx=[250, 90], q_lens=[1, 1], mode=NO)
    kc, vc, _, _ = build_cache(w)
    s_k, s_v = np.float32(0.03125), np.float32(0.0234375)
    ks = np.full(w.num_blocks * 128, s_k, np.float32)
    vs = np.full(w.num_blocks * 128, s_v, np.float32)
    a = att.attention_ref(w.q, kc, vc, ks, vs, w.block_table, w.ctx, None, None, PT, 1)
    b = att.attention_ref(w.q, kc, vc, np.array([s_k]), np.array([s_v]), w.block_table, w.ctx,
                          None, None, SC, 1)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(7)
    n = 700
    k = rng.standard_normal((n, 128))
    v = rng.standard_normal((n, 128))
    qv = rng.standard_normal(128)
    sm = 1 / math.sqrt(128)
    whole = att._softmax_attend(qv, k, v, sm)
    for trial in range(20):
        cuts = np.sort(rng.integers(0, n + 1, size=rng.integers(1, 9)))
        bounds = np.concatenate([[0], cuts, [n]])
        parts = [att.attention_partial(qv, k[a:b], v[a:b], sm) for a, b in zip(bounds[:-1], bounds[1:])]
        np.testing.assert_allclose(att.lse_merge(parts), whole, rtol=1e-12, atol=1e-14)
    assert np.array_equal(att.lse_merge([att.attention_partial(qv, k[:0], v[:0], sm)] * 3),
                          np.zeros(128))


def test_multirow_row_equals_single_row_at_shifted_cutoff():
    """Row i of a q_len-L request equals a q_len-1 decode with context
    ctx - L + i + 1 (the cutoff rule)."""
    w = wl.small_case(seed=27, ctx=[300, 261], q_lens=[4, 3], ragged=True)
    cache = build_cache(w)
    out = run_ref(w, cache)
    starts = w.row_start
    for b in range(2):
        L = int(w.q_lens[b])
        for i in range(L):
            r = int(starts[b] + i)
            ctx1 = np.array([int(w.ctx[b]) - L + i + 1], np.int32)
            single = att.attention_ref(w.q[r:r + 1], cache[0], cache[1], cache[2], cache[3],
                                       w.block_table[b:b + 1], ctx1, None, None, PT, 1)
            assert np.array_equal(single[0], out[r])


def test_sparse_with_all_pages_equals_dense_and_order_free():
    w = wl.small_case(seed=28, ctx=[600, 390], q_lens=[1, 1])
    cache = build_cache(w)
    dense = run_ref(w, cache)
    W = w.W
    sp = np.full((2, W), -1, np.int32)
    for b in range(2):
        npg = -(-int(w.ctx[b]) // 128)
        sp[b, :npg] = np.random.default_rng(b).permutation(npg)
    kc, vc, ks, vs = cache
    sparse = att.attention_ref(w.q, kc, vc, ks, vs, w.block_table, w.ctx, None, sp, PT, 1)
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_torch_sdpa():
    w = wl.small_case(seed=29, ctx=[200, 333], q_lens=[1, 1], Hkv=2)
    cache = build_cache(w)
    kc, vc, ks, vs = cache
    out = run_ref(w, cache)
    for b in range(2):
        c = int(w.ctx[b])
        K = np.zeros((2, c, 128))
        V = np.zeros((2, c, 128))
        for h in range(2):
            for t in range(c):
                P = int(w.block_table[b, t // 128])
                o = t % 128
                base = int(layout.block_base(P, h, 2))
                s = layout.scale_index(P, h, o, 2)
                K[h, t] = e4m3.decode(kc[base + layout.k_offset(o, np.arange(128))]) * float(ks[s])
                V[h, t] = e4m3.decode(vc[base + layout.v_offset(o, np.arange(128))]) * float(vs[s])
        Kr = torch.from_numpy(np.repeat(K, 16, axis=0))[None]          # [1, 32, c, 128]
        Vr = torch.from_numpy(np.repeat(V, 16, axis=0))[None]
        Q = torch.from_numpy(w.q[b].astype(np.float64))[None, :, None, :]  # [1, 32, 1, 128]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr)[0, :, 0].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-10, atol=1e-12)


def test_empty_context_gives_zero():
    w = wl.small_case(seed=30, ctx=[0, 50], q_lens=[1, 1], pool=4, W=1)
    cache = build_cache(w)
    out = run_ref(w, cache)
    assert np.array_equal(out[0], np.zeros((16, 128)))
    assert np.all(np.isfinite(out[1]))
