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


# ---------------------------------------------------------------------------
# The per-token quotient is one IEEE fp32 division, not a multiply by a
# rounded reciprocal.  Each case below puts x exactly on an e4m3 rounding
# midpoint of x / scale, with scale = amax / 448 exact in fp32 and not a
# power of two, so the division lands on the tie (rounded to even) while
# x * fl32(1 / scale) lands one fp32 ulp to the odd side.  The expected codes
# come from exact rational arithmetic (tests/exact_rational.py); the cases
# were found by a search over 10-bit scale significands.
from fractions import Fraction  # noqa: E402

from exact_rational import e4m3_code, quantize_by_reciprocal, quantize_exact, round_f32  # noqa: E402

# (scale significand / 512, power of two, midpoint of x / scale)
DIVISION_CASES = [
    (943, -1, Fraction(21, 16)),   # 1.3125: tie -> 1.25 (0x3A); reciprocal lands above -> 0x3B
    (881, -7, Fraction(21, 16)),
    (933, -10, Fraction(23, 16)),  # 1.4375: tie -> 1.5 (0x3C); reciprocal lands below -> 0x3B
    (948, -9, Fraction(23, 16)),
    (874, -5, Fraction(27, 8)),    # 3.375: tie -> 3.5 (0x46); reciprocal lands below -> 0x45
]


def test_exact_rational_helpers():
    """The exact models agree with hand-worked values and with torch's own
    float32 / float8_e4m3fn conversions."""
    import torch
    F = Fraction
    assert e4m3_code(F(17, 16)) == 0x38 and e4m3_code(F(19, 16)) == 0x3A
    assert e4m3_code(F(1, 1024)) == 0x00 and e4m3_code(F(3, 1024)) == 0x02
    assert e4m3_code(F(448)) == 0x7E and e4m3_code(F(470)) == 0x7E and e4m3_code(F(-1, 512)) == 0x81
    assert round_f32(F(1, 3)) == F(11184811, 2 ** 25)
    assert round_f32(F(2 ** 24 + 1)) == F(2 ** 24)          # tie to even
    assert round_f32(F(2 ** 24 + 3)) == F(2 ** 24 + 4)
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(400) * 50, rng.standard_normal(100) * 0.01])
    f32 = vals.astype(np.float32)
    for v, r in zip(vals.tolist(), f32.tolist()):
        assert round_f32(F(v)) == F(r)
    ref = torch.from_numpy(np.clip(f32, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, c in zip(f32.tolist(), ref.tolist()):
        assert e4m3_code(F(v)) == c, v


@pytest.mark.parametrize("m,e,mid", DIVISION_CASES)
def test_per_token_quotient_is_a_division(m, e, mid):
    s = Fraction(m, 512) * Fraction(2) ** e
    amax, x = 448 * s, mid * s
    # every input is an fp32 value, and amax / 448 is exactly s
    assert round_f32(amax) == amax and round_f32(x) == x
    s_div, want = quantize_exact(x, amax)
    s_rec, other = quantize_by_reciprocal(x, amax)
    assert s_div == s == s_rec
    assert want != other, "case does not tell division from reciprocal"
    row = np.zeros((1, 1, 128), dtype=np.float32)
    row[0, 0, 0] = float(amax)
    row[0, 0, 1] = float(x)
    row[0, 0, 2] = -float(x)
    row[0, 0, 3] = -float(amax)
    codes, scale = writer.quantize_rows(row, PT)
    assert Fraction(float(scale[0, 0])) == s
    assert codes[0, 0, 1] == want and codes[0, 0, 2] == (want | 0x80)
    assert codes[0, 0, 0] == 0x7E and codes[0, 0, 3] == 0xFE
    # and through the whole writer (layout and scale store)
    kc, vc, ks, vs = _fresh(1, 1)
    writer.quant_write_ref(row, row, np.array([77]), kc, vc, ks, vs, PT, 1)
    got = _read_back(kc, 0, 0, 77, 1, "k")
    assert got[1] == want and got[2] == (want | 0x80)
    assert Fraction(float(ks[layout.scale_index(0, 0, 77, 1)])) == s
