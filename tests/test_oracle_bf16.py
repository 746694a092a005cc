"""Pins for the oracle's bf16 element code and the BF16-cache paths of the
writer and the attention: decode and encode against torch's own bfloat16
conversion (round to nearest even), hand-worked ties and overflow, the
writer storing bf16 inputs unchanged, and attention over a bf16 cache
against the loop-only brute force and torch's fp64 SDPA."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as att
from oracle import bf16, layout, writer


def test_decode_every_pattern_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16.decode(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, 1.17549435e-38],
                 np.float32),
    ])
    ours = bf16.encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN with its sign
    d = bf16.decode(ours[nan])
    assert np.all(np.isnan(d))
    assert np.array_equal(np.signbit(x[nan]), (ours[nan] & 0x8000) != 0)


def test_encode_hand_worked_ties_and_overflow():
    # 1 + 2^-8 lies halfway between 1 (mantissa 0, even) and 1 + 2^-7: -> 1
    assert bf16.encode(np.float32(1 + 2 ** -8)) == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): -> 1 + 2^-6
    assert bf16.encode(np.float32(1 + 3 * 2 ** -8)) == 0x3F82
    # just above the tie rounds up
    assert bf16.encode(np.float32(1 + 2 ** -8 + 2 ** -20)) == 0x3F81
    # the largest float rounds past the largest bf16: infinity
    assert bf16.encode(np.float32(3.4028235e38)) == 0x7F80
    assert bf16.encode(np.float32(-2.0)) == 0xC000


def _fresh(nb, Hkv, fill=0x7FC1):
    kc = np.full(nb * Hkv * 16384, fill, dtype=np.uint16)
    return kc, kc.copy()


@pytest.mark.parametrize("Hkv", [1, 2])
def test_writer_stores_bf16_inputs_unchanged(Hkv):
    rng = np.random.default_rng(3)
    T, nb = 40, 3
    k = wl.bf16_round(rng.standard_normal((T, Hkv, 128)).astype(np.float32) * 5)
    v = wl.bf16_round(rng.standard_normal((T, Hkv, 128)).astype(np.float32))
    slots = rng.permutation(nb * 128)[:T].astype(np.int64)
    slots[7] = -1
    kc, vc = _fresh(nb, Hkv)
    writer.write_bf16_ref(k, v, slots, kc, vc, Hkv)
    touched = np.zeros(kc.size, bool)
    for t in range(T):
        if slots[t] < 0:
            continue
        P, o = divmod(int(slots[t]), 128)
        for h in range(Hkv):
            base = (P * Hkv + h) * 16384
            ki = base + layout.k_offset_bf16(o, np.arange(128))
            vi = base + layout.v_offset_bf16(o, np.arange(128))
            assert np.array_equal(bf16.decode(kc[ki]), k[t, h].astype(np.float64))
            assert np.array_equal(bf16.decode(vc[vi]), v[t, h].astype(np.float64))
            touched[ki] = True
    assert np.all(kc[~touched] == 0x7FC1)
    assert touched.sum() == (T - 1) * Hkv * 128


def test_writer_rounds_fp32_to_nearest_even():
    k = np.full((1, 1, 128), 1 + 3 * 2 ** -8, np.float32)
    v = np.full((1, 1, 128), -(1 + 2 ** -8), np.float32)
    kc, vc = _fresh(1, 1)
    writer.write_bf16_ref(k, v, np.array([0], np.int64), kc, vc, 1)
    assert kc[layout.k_offset_bf16(0, 5)] == 0x3F82
    assert vc[layout.v_offset_bf16(0, 5)] == 0xBF80


def build_bf16_cache(w, poison=True):
    rng = np.random.default_rng(w.seed + 98)
    n = w.num_blocks * w.Hkv * 16384
    if poison:
        # finite poison: large values a missed mask would not hide
        kc = bf16.encode(rng.uniform(-300, 300, size=n).astype(np.float32))
        vc = bf16.encode(rng.uniform(-300, 300, size=n).astype(np.float32))
    else:
        kc = np.zeros(n, np.uint16)
        vc = kc.copy()
    for b in range(w.B):
        k, v, s = w.request_kv(b)
        writer.write_bf16_ref(k, v, s, kc, vc, w.Hkv)
    return kc, vc


TINY = [
    dict(seed=41, ctx=[1, 5, 130], q_lens=[1, 1, 1], Hkv=1),
    dict(seed=42, ctx=[7, 140], q_lens=[2, 2], Hkv=2),
    dict(seed=43, ctx=[9, 3, 131], q_lens=[3, 1, 2], Hkv=1, ragged=True),
]


@pytest.mark.parametrize("cfg", TINY)
def test_bf16_attention_matches_bruteforce(cfg):
    w = wl.small_case(**cfg)
    kc, vc = build_bf16_cache(w)
    ref = att.attention_ref(w.q, kc, vc, None, None, w.block_table, w.ctx, w.cu, None,
                            att.NONE, w.Hkv, kv_dtype="bf16")
    bru = att.attention_bruteforce(w.q, kc, vc, None, None, w.block_table, w.ctx, w.cu, None,
                                   att.NONE, w.Hkv, kv_dtype="bf16")
    np.testing.assert_allclose(ref, bru, rtol=1e-12, atol=1e-13)


def test_bf16_sparse_matches_bruteforce():
    w = wl.small_case(seed=44, ctx=[700, 300], q_lens=[1, 1], sparse_topk=3)
    kc, vc = build_bf16_cache(w)
    args = (w.q, kc, vc, None, None, w.block_table, w.ctx, None, w.sparse, att.NONE, 1)
    ref = att.attention_ref(*args, kv_dtype="bf16")
    bru = att.attention_bruteforce(*args, kv_dtype="bf16")
    np.testing.assert_allclose(ref, bru, rtol=1e-12, atol=1e-13)


def test_bf16_gqa_equals_torch_sdpa():
    """K/V read back through the layout, repeated per query head, into
    torch's fp64 scaled_dot_product_attention."""
    w = wl.small_case(seed=45, ctx=[200, 333], q_lens=[1, 1], Hkv=2)
    kc, vc = build_bf16_cache(w)
    out = att.attention_ref(w.q, kc, vc, None, None, w.block_table, w.ctx, None, None,
                            att.NONE, 2, kv_dtype="bf16")
    for b in range(2):
        c = int(w.ctx[b])
        K = np.zeros((2, c, 128))
        V = np.zeros((2, c, 128))
        for h in range(2):
            for t in range(c):
                P = int(w.block_table[b, t // 128])
                base = (P * 2 + h) * 16384
                K[h, t] = bf16.decode(kc[base + layout.k_offset_bf16(t % 128, np.arange(128))])
                V[h, t] = bf16.decode(vc[base + layout.v_offset_bf16(t % 128, np.arange(128))])
        # the cache holds the generator's values rounded to bf16
        kk, vv, _ = w.request_kv(b)
        np.testing.assert_array_equal(K.transpose(1, 0, 2), wl.bf16_round(kk).astype(np.float64))
        Kr = torch.from_numpy(np.repeat(K, 16, axis=0))[None]
        Vr = torch.from_numpy(np.repeat(V, 16, axis=0))[None]
        Q = torch.from_numpy(w.q[b].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr)[0, :, 0].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-10, atol=1e-12)


def test_bf16_one_token_context_returns_v():
    w = wl.small_case(seed=46, ctx=[1], q_lens=[1])
    kc, vc = build_bf16_cache(w)
    out = att.attention_ref(w.q, kc, vc, None, None, w.block_table, w.ctx, None, None,
                            att.NONE, 1, kv_dtype="bf16")
    _, v, _ = w.request_kv(0)
    np.testing.assert_array_equal(out[0], np.repeat(wl.bf16_round(v[0]).astype(np.float64), 16, axis=0))
