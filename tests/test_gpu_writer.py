"""GPU parity of kv_quant_write against the oracle's writer: every byte of
both caches and every scale bit-exact, untouched slots untouched."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl
from oracle import writer as owr

from harness import GpuCase, oracle_cache, poison_arrays

pytestmark = pytest.mark.gpu


def _cmp_cache(case, w, cache):
    kc, vc, ks, vs, _, _ = cache
    assert np.array_equal(case.kc.view(torch.uint8).cpu().numpy().reshape(-1), kc), "K bytes differ"
    assert np.array_equal(case.vc.view(torch.uint8).cpu().numpy().reshape(-1), vc), "V bytes differ"
    if w.mode == wl.PER_TOKEN:
        assert np.array_equal(case.ks.cpu().numpy().reshape(-1).view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(case.vs.cpu().numpy().reshape(-1).view(np.uint32), vs.view(np.uint32))


@pytest.mark.parametrize("kw", [
    dict(seed=101, ctx=[300, 513], q_lens=[1, 1]),
    dict(seed=102, ctx=[1, 129, 1000], q_lens=[1, 1, 1], Hkv=2),
    dict(seed=103, ctx=[200, 77], q_lens=[2, 3], ragged=True, mode=wl.SCALAR),
    dict(seed=104, ctx=[260], q_lens=[1], mode=wl.NONE),
    dict(seed=105, ctx=[700, 300], q_lens=[1, 1], Hkv=3, sparse_topk=2),
])
def test_writer_bit_exact(kw):
    w = wl.small_case(**kw)
    print("writer case", w.name, flush=True)
    case = GpuCase(w)
    torch.cuda.synchronize()
    _cmp_cache(case, w, oracle_cache(w))


def test_writer_bf16_inputs_and_f8_label():
    w = wl.small_case(seed=106, ctx=[333, 64], q_lens=[1, 1], Hkv=2)
    case = GpuCase(w, kv_dtype=torch.float8_e4m3fn, in_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    kc, vc, ks, vs = poison_arrays(w)
    for b in range(w.B):
        k, v, s = w.request_kv(b)
        owr.quant_write_ref(wl.bf16_round(k), wl.bf16_round(v), s, kc, vc, ks, vs, w.mode, w.Hkv)
    _cmp_cache(case, w, (kc, vc, ks, vs, ks, vs))


def test_writer_edge_values_and_skipped_slots():
    """Zero rows, signed zeros, tiny and huge values, saturation in scalar
    mode, infinities, skipped (-1) and out-of-range slots."""
    dev = torch.device("cuda:0")
    Hkv, nb = 2, 3
    rng = np.random.default_rng(7)
    T = 12
    k = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    k[0] = 0.0
    k[0, 0, ::3] = -0.0
    k[1] *= np.float32(1e-38)           # scale becomes an fp32 subnormal
    k[2] *= np.float32(1e30)
    v[3, 1, :] = np.float32(2.0 ** -12)  # rounds to subnormal codes
    k[4, 0, 5] = np.float32(448.0 * 3)   # dominant element
    slots = np.array([0, 5, 130, 131, 255, -1, 3 * 128, 10, 11, 12, 200, 201], dtype=np.int64)
    for mode, sc in ((wl.PER_TOKEN, None), (wl.SCALAR, np.float32(0.01)), (wl.NONE, None)):
        kk, vv = k.copy(), v.copy()
        if mode != wl.PER_TOKEN:
            kk[2] = np.clip(kk[2], -1e30, 1e30)
            kk[5, 0, :4] = [np.inf, -np.inf, 500.0, -460.0]
        kc0 = rng.integers(0, 256, size=nb * Hkv * 16384, dtype=np.uint8)
        vc0 = rng.integers(0, 256, size=nb * Hkv * 16384, dtype=np.uint8)
        ks0 = np.full(nb * Hkv * 128, -3.0, np.float32)
        kc_g = torch.from_numpy(kc0.copy()).to(dev).view(nb, Hkv, 16384)
        vc_g = torch.from_numpy(vc0.copy()).to(dev).view(nb, Hkv, 16384)
        if mode == wl.SCALAR:
            ks_g = torch.tensor([sc], device=dev)
            vs_g = torch.tensor([sc], device=dev)
        elif mode == wl.PER_TOKEN:
            ks_g = torch.from_numpy(ks0.copy()).to(dev).view(nb, Hkv, 128)
            vs_g = torch.from_numpy(ks0.copy()).to(dev).view(nb, Hkv, 128)
        else:
            ks_g = vs_g = None
        pa.kv_quant_write(torch.from_numpy(kk).to(dev), torch.from_numpy(vv).to(dev),
                          torch.from_numpy(slots).to(dev), kc_g, vc_g, ks_g, vs_g, mode)
        torch.cuda.synchronize()
        kc, vc, ks, vs = kc0.copy(), vc0.copy(), ks0.copy(), ks0.copy()
        if mode == wl.SCALAR:
            owr.quant_write_ref(kk, vv, slots, kc, vc, np.array([sc]), np.array([sc]), mode, Hkv)
        else:
            owr.quant_write_ref(kk, vv, slots, kc, vc, ks, vs, mode, Hkv)
        assert np.array_equal(kc_g.cpu().numpy().reshape(-1), kc), mode
        assert np.array_equal(vc_g.cpu().numpy().reshape(-1), vc), mode
        if mode == wl.PER_TOKEN:
            assert np.array_equal(ks_g.cpu().numpy().reshape(-1).view(np.uint32), ks.view(np.uint32))
            assert np.array_equal(vs_g.cpu().numpy().reshape(-1).view(np.uint32), vs.view(np.uint32))


def test_writer_exhaustive_codes_in_none_mode():
    """Every fp32 bit pattern class that matters: all bf16 patterns plus
    e4m3 midpoints +-1 ulp, written in no-scale mode, must give the oracle's
    codes."""
    from oracle import e4m3
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    t = e4m3.decode_table()[:127]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    vals = np.concatenate([bits, mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf)), -mids])
    vals = vals[~np.isnan(vals)]
    n = (len(vals) + 127) // 128 * 128
    vals = np.concatenate([vals, np.zeros(n - len(vals), np.float32)])
    T = n // 128
    x = vals.reshape(T, 1, 128)
    nb = (T + 127) // 128
    dev = torch.device("cuda:0")
    kc_g = torch.zeros(nb, 1, 16384, dtype=torch.uint8, device=dev)
    vc_g = torch.zeros_like(kc_g)
    slots = np.arange(T, dtype=np.int64)
    xt = torch.from_numpy(x).to(dev)
    pa.kv_quant_write(xt, xt, torch.from_numpy(slots).to(dev), kc_g, vc_g, None, None, wl.NONE)
    torch.cuda.synchronize()
    kc = np.zeros(nb * 16384, np.uint8)
    vc = kc.copy()
    owr.quant_write_ref(x, x, slots, kc, vc, None, None, wl.NONE, 1)
    assert np.array_equal(kc_g.cpu().numpy().reshape(-1), kc)
    assert np.array_equal(vc_g.cpu().numpy().reshape(-1), vc)


@pytest.mark.parametrize("seed", list(range(801, 833)))
def test_writer_random_calls_bit_exact(seed):
    """Seeded random writer calls: 1-300 tokens, 1-4 KV heads, fp32 or bf16
    inputs, every scale mode, per-token magnitudes from 1e-30 to 1e30 with
    all-zero tokens, and slots that are distinct, skipped (-1) or past the
    pool; every byte and scale bit against the oracle's writer."""
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    T = int(rng.integers(1, 301))
    Hkv = int(rng.integers(1, 5))
    nb = int(rng.integers(1, 5))
    mode = [wl.PER_TOKEN, wl.SCALAR, wl.NONE][int(rng.integers(0, 3))]
    bf16_in = bool(rng.random() < 0.4)
    mag = (10.0 ** rng.uniform(-30, 30, size=(T, Hkv, 1))) if mode == wl.PER_TOKEN else \
        (10.0 ** rng.uniform(-3, 3, size=(T, Hkv, 1)))
    k = (rng.standard_normal((T, Hkv, 128)) * mag).astype(np.float32)
    v = (rng.standard_normal((T, Hkv, 128)) * mag).astype(np.float32)
    k[rng.random(T) < 0.05] = 0.0
    if bf16_in:
        k, v = wl.bf16_round(k), wl.bf16_round(v)
    slots = rng.permutation(nb * 128)[:T].astype(np.int64)
    if T > nb * 128:
        slots = np.concatenate([slots, np.full(T - nb * 128, -1, np.int64)])
    slots[rng.random(T) < 0.1] = -1
    slots[rng.random(T) < 0.05] = nb * 128 + int(rng.integers(0, 1000))
    print("writer random", seed, "T", T, "Hkv", Hkv, "nb", nb, "mode", mode, "bf16", bf16_in, flush=True)
    kc0 = rng.integers(0, 256, size=nb * Hkv * 16384, dtype=np.uint8)
    vc0 = rng.integers(0, 256, size=nb * Hkv * 16384, dtype=np.uint8)
    s0 = np.full(nb * Hkv * 128, -3.0, np.float32)
    kc_g = torch.from_numpy(kc0.copy()).to(dev).view(nb, Hkv, 16384)
    vc_g = torch.from_numpy(vc0.copy()).to(dev).view(nb, Hkv, 16384)
    if mode == wl.SCALAR:
        sk, sv = np.float32(rng.uniform(1e-3, 1)), np.float32(rng.uniform(1e-3, 1))
        ks_g, vs_g = torch.tensor([sk], device=dev), torch.tensor([sv], device=dev)
    elif mode == wl.PER_TOKEN:
        ks_g = torch.from_numpy(s0.copy()).to(dev).view(nb, Hkv, 128)
        vs_g = torch.from_numpy(s0.copy()).to(dev).view(nb, Hkv, 128)
    else:
        ks_g = vs_g = None
    tin = torch.bfloat16 if bf16_in else torch.float32
    pa.kv_quant_write(torch.from_numpy(k).to(dev).to(tin), torch.from_numpy(v).to(dev).to(tin),
                      torch.from_numpy(slots).to(dev), kc_g, vc_g, ks_g, vs_g, mode)
    torch.cuda.synchronize()
    kc, vc, ks, vs = kc0.copy(), vc0.copy(), s0.copy(), s0.copy()
    if mode == wl.SCALAR:
        owr.quant_write_ref(k, v, slots, kc, vc, np.array([sk]), np.array([sv]), mode, Hkv)
    else:
        owr.quant_write_ref(k, v, slots, kc, vc, ks, vs, mode, Hkv)
    assert np.array_equal(kc_g.cpu().numpy().reshape(-1), kc)
    assert np.array_equal(vc_g.cpu().numpy().reshape(-1), vc)
    if mode == wl.PER_TOKEN:
        assert np.array_equal(ks_g.cpu().numpy().reshape(-1).view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(vs_g.cpu().numpy().reshape(-1).view(np.uint32), vs.view(np.uint32))


def test_writer_quotient_is_a_division():
    """The rows of the oracle's division pins (x on an e4m3 midpoint of
    x / scale, where a reciprocal multiply would round the other way),
    through the GPU writer: codes and scales equal the exact-rational ones."""
    from fractions import Fraction

    from exact_rational import quantize_exact
    from test_oracle_writer import DIVISION_CASES
    dev = torch.device("cuda:0")
    T = len(DIVISION_CASES)
    k = np.zeros((T, 1, 128), np.float32)
    want = []
    for t, (m, e, mid) in enumerate(DIVISION_CASES):
        s = Fraction(m, 512) * Fraction(2) ** e
        k[t, 0, 0], k[t, 0, 1], k[t, 0, 2] = float(448 * s), float(mid * s), -float(mid * s)
        want.append((s, quantize_exact(mid * s, 448 * s)[1]))
    slots = np.arange(T, dtype=np.int64) * 7
    kc_g = torch.zeros(1, 1, 16384, dtype=torch.uint8, device=dev)
    vc_g = torch.zeros_like(kc_g)
    ks_g = torch.zeros(1, 1, 128, dtype=torch.float32, device=dev)
    vs_g = torch.zeros_like(ks_g)
    kt = torch.from_numpy(k).to(dev)
    pa.kv_quant_write(kt, kt, torch.from_numpy(slots).to(dev), kc_g, vc_g, ks_g, vs_g, wl.PER_TOKEN)
    torch.cuda.synchronize()
    kc = np.zeros(16384, np.uint8)
    vc = kc.copy()
    ks = np.zeros(128, np.float32)
    vs = ks.copy()
    owr.quant_write_ref(k, k, slots, kc, vc, ks, vs, wl.PER_TOKEN, 1)
    assert np.array_equal(kc_g.cpu().numpy().reshape(-1), kc)
    assert np.array_equal(ks_g.cpu().numpy().reshape(-1).view(np.uint32), ks.view(np.uint32))
    from oracle import layout as olay
    got = kc_g.cpu().numpy().reshape(-1)
    gs = ks_g.cpu().numpy().reshape(-1)
    for t, (s, code) in enumerate(want):
        o = int(slots[t])
        codes = got[olay.k_offset(o, np.arange(128))]
        assert Fraction(float(gs[o])) == s
        assert codes[1] == code and codes[2] == (code | 0x80), (t, codes[:3], code)
