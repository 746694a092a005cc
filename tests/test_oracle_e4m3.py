"""Pins for the oracle's e4m3fn codec against things other than itself:
torch's CPU float8_e4m3fn cast (a library routine), the format's printed
extremes, hand-worked ties, and two independent encoders."""

import numpy as np
import pytest
import torch

from oracle import e4m3


def test_decode_matches_torch_all_256_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mine = e4m3.decode_table()
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(mine))
    assert set(np.nonzero(nan_ref)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], mine[~nan_ref])
    # signed zero
    assert np.signbit(mine[0x80]) and not np.signbit(mine[0x00])


def test_decode_extremes():
    t = e4m3.decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0                # e = 7, m = 0
    finite = t[np.isfinite(t)]
    assert np.abs(finite).max() == 448.0


def _all_bf16_as_f32():
    bits = (np.arange(65536, dtype=np.uint32) << 16)
    return bits.view(np.float32)


def _midpoints():
    t = e4m3.decode_table()[:127]
    mids = (t[:-1] + t[1:]) / 2.0                    # exact in fp64, representable in fp32
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(-np.inf))
    v = np.concatenate([m32, up, dn, t.astype(np.float32)])
    return np.concatenate([v, -v])


def test_hand_worked_ties():
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): goes to 0x38.
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even): goes to 0x3A.
    # 2^-10 is halfway between 0 and 2^-9: goes to 0x00; 3*2^-10 goes to 0x02.
    y = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 1e30, -0.0, -2.0 ** -12],
                 dtype=np.float32)
    want = np.array([0x38, 0x3A, 0x00, 0x02, 0x7E, 0x7E, 0x80, 0x80], dtype=np.uint8)
    assert np.array_equal(e4m3.encode_bruteforce(y), want)
    assert np.array_equal(e4m3.encode_closed_form(y), want)


def test_encoders_agree_on_bf16_patterns_and_midpoints():
    y = np.concatenate([_all_bf16_as_f32(), _midpoints()])
    a = e4m3.encode_bruteforce(y)
    b = e4m3.encode_closed_form(y)
    # NaN inputs: both give 0x7F with the input's sign
    assert np.array_equal(a, b)


def test_closed_form_matches_torch_cast_on_clamped_values():
    rng = np.random.default_rng(1)
    y = np.concatenate([
        _all_bf16_as_f32(),
        _midpoints(),
        rng.standard_normal(1_000_000).astype(np.float32) * np.float32(30.0),
        (rng.random(200_000) * 2 - 1).astype(np.float32) * np.float32(2.0 ** -6),
    ])
    y = y[np.isfinite(y)]
    clamped = np.clip(y, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode_closed_form(y)
    assert np.array_equal(got, ref)


def test_bruteforce_matches_torch_on_random_sample():
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(20000) * 50).astype(np.float32)
    ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode_bruteforce(y), ref)


def test_saturation_and_nan():
    y = np.array([448.0, 449.0, 480.0, np.inf, -np.inf, np.nan, -np.nan], dtype=np.float32)
    got = e4m3.encode_closed_form(y)
    assert got[:5].tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert (got[5] & 0x7F) == 0x7F and (got[6] & 0x7F) == 0x7F


def test_round_trip_error_bound():
    """|dec(enc(y)) - y| <= half a code spacing: 2^-4 |y| in the normal
    range, 2^-10 in the subnormal range (format arithmetic)."""
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(200000) * 40).astype(np.float32)
    y = y[np.abs(y) < 448]
    back = e4m3.decode(e4m3.encode(y))
    err = np.abs(back - y.astype(np.float64))
    bound = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** -4 * np.abs(y.astype(np.float64)), 2.0 ** -10)
    assert np.all(err <= bound)
