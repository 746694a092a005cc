"""Pins for the oracle's cache writer: the amax element lands on +-448, the
round trip stays within the e4m3 error bound, zero rows and skipped slots
behave as defined, and nothing outside the named slots changes."""

import numpy as np
import pytest

from oracle import e4m3, layout, writer

PT, SC, NO = writer.PER_TOKEN, writer.SCALAR, writer.NONE


def _fresh(num_blocks, Hkv, fill=0xA5):
    kc = np.full(num_blocks * Hkv * 16384, fill, dtype=np.uint8)
    vc = kc.copy()
    ks = np.full(num_blocks * Hkv * 128, -7.0, dtype=np.float32)
    return kc, vc, ks, ks.copy()


def _read_back(cache, page, head, slot, Hkv, kind):
    base = int(layout.block_base(page, head, Hkv))
    f = layout.k_offset if kind == "k" else layout.v_offset
    return cache[base + f(slot, np.arange(128))]


@pytest.mark.parametrize("Hkv", [1, 2])
def test_amax_maps_to_448_and_round_trip(Hkv):
    rng = np.random.default_rng(0)
    T, nb = 50, 3
    k = rng.standard_normal((T, Hkv, 128)).astype(np.float32) * 3
    v = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    slots = rng.choice(nb * 128, size=T, replace=False).astype(np.int64)
    kc, vc, ks, vs = _fresh(nb, Hkv)
    writer.quant_write_ref(k, v, slots, kc, vc, ks, vs, PT, Hkv)
    for t in range(T):
        p, o = divmod(int(slots[t]), 128)
        for h in range(Hkv):
            for x, cache, sc, kind in ((k, kc, ks, "k"), (v, vc, vs, "v")):
                codes = _read_back(cache, p, h, o, Hkv, kind)
                scale = sc[layout.scale_index(p, h, o, Hkv)]
                row = x[t, h]
                amax = np.abs(row).max()
                assert scale == np.float32(amax / np.float32(448))
                i = int(np.argmax(np.abs(row)))
                assert codes[i] == (0xFE if row[i] < 0 else 0x7E)
                # no code above 448 in magnitude, none NaN
                assert np.all((codes & 0x7F) <= 0x7E)
                back = e4m3.decode(codes) * float(scale)
                err = np.abs(back - row.astype(np.float64))
                y = np.abs(row.astype(np.float64)) / float(scale)
                bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * y, 2.0 ** -10) * float(scale)
                assert np.all(err <= bound * (1 + 2.0 ** -20) + 1e-30)


def test_sentinel_and_skip():
    rng = np.random.default_rng(1)
    Hkv, nb = 2, 4
    k = rng.standard_normal((6, Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((6, Hkv, 128)).astype(np.float32)
    slots = np.array([5, -1, 130, 511, 512 * 7, 300], dtype=np.int64)  # -1 and out-of-range skipped
    kc, vc, ks, vs = _fresh(nb, Hkv)
    kc0, vc0, ks0 = kc.copy(), vc.copy(), ks.copy()
    writer.quant_write_ref(k, v, slots, kc, vc, ks, vs, PT, Hkv)
    touched = set()
    for s in (5, 130, 511, 300):
        p, o = divmod(s, 128)
        for h in range(Hkv):
            base = int(layout.block_base(p, h, Hkv))
            touched |= set((base + layout.k_offset(o, np.arange(128))).tolist())
    changed = np.nonzero(kc != kc0)[0]
    assert set(changed.tolist()) <= touched
    untouched = np.ones(kc.size, bool)
    untouched[list(touched)] = False
    assert np.array_equal(kc[untouched], kc0[untouched])
    sc_changed = set(np.nonzero(ks != ks0)[0].tolist())
    want = {int(layout.scale_index(s // 128, h, s % 128, Hkv)) for s in (5, 130, 511, 300)
            for h in range(Hkv)}
    assert sc_changed == want


def test_zero_row_and_signed_zero():
    Hkv = 1
    k = np.zeros((1, 1, 128), dtype=np.float32)
    k[0, 0, ::2] = -0.0
    v = np.zeros((1, 1, 128), dtype=np.float32)
    kc, vc, ks, vs = _fresh(1, Hkv)
    writer.quant_write_ref(k, v, np.array([3]), kc, vc, ks, vs, PT, Hkv)
    codes = _read_back(kc, 0, 0, 3, Hkv, "k")
    assert ks[3] == 0.0
    assert np.array_equal(codes, np.where(np.signbit(k[0, 0]), 0x80, 0x00).astype(np.uint8))


def test_scalar_and_none_modes():
    rng = np.random.default_rng(2)
    k = (rng.standard_normal((8, 1, 128)) * 5).astype(np.float32)
    v = (rng.standard_normal((8, 1, 128)) * 5).astype(np.float32)
    slots = np.arange(8, dtype=np.int64) * 3
    s = np.array([0.01], dtype=np.float32)
    kc, vc, _, _ = _fresh(1, 1)
    writer.quant_write_ref(k, v, slots, kc, vc, s, s, SC, 1)
    for t in range(8):
        codes = _read_back(kc, 0, 0, int(slots[t]), 1, "k")
        want = e4m3.encode_bruteforce((k[t, 0] / np.float32(0.01)).astype(np.float32))
        assert np.array_equal(codes, want)
        # |x| > 4.48 saturates to 448 at scale 0.01
        big = np.abs(k[t, 0]) / np.float32(0.01) >= 448
        assert np.all((codes[big] & 0x7F) == 0x7E)
    kc, vc, _, _ = _fresh(1, 1)
    writer.quant_write_ref(k, v, slots, kc, vc, None, None, NO, 1)
    for t in range(8):
        codes = _read_back(vc, 0, 0, int(slots[t]), 1, "v")
        assert np.array_equal(codes, e4m3.encode_bruteforce(v[t, 0]))
