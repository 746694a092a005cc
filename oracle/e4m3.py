"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format definition.

Test infrastructure only (see ``oracle/__init__``).

The pages store the KV cache as FP8 bytes whose true dtype is
``torch.float8_e4m3fn`` (ROCm/ATOM pull request 2122, "fix(minimax-m3):
unblock fp8 KV cache ...", section 1: the bytes are fp8 even where the
tensor is labelled uint8).  The format (OCP 8-bit floating point
specification, E4M3 variant without infinities):

* bit 7 sign s, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m;
* e == 0: subnormal, value (-1)^s * 2^-6 * m/8 (smallest 2^-9);
* 1 <= e <= 15 and not (e == 15 and m == 7): value (-1)^s * 2^(e-7) * (1+m/8),
  so the largest finite magnitude is 2^8 * 1.75 = 448;
* e == 15 and m == 7 (bytes 0x7F, 0xFF): NaN.  There is no infinity.

Encoding (the pages do not state a rounding rule; the reading taken here):
round to nearest, ties to the even code, and saturate: any magnitude at or
above 448 (infinity included) maps to 448; NaN maps to 0x7F with the input's
sign bit; the sign of zero is kept.
"""

import numpy as np

MAX_FINITE = 448.0
MIN_SUBNORMAL = 2.0 ** -9


def decode_byte(c: int) -> float:
    """Value of one e4m3fn byte, straight from the bit fields."""
    c = int(c) & 0xFF
    s = -1.0 if (c >> 7) else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (2.0 ** -6) * (m / 8.0)
    return s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


def decode_table() -> np.ndarray:
    """All 256 byte values decoded to fp64 (index = byte)."""
    return np.array([decode_byte(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of e4m3fn bytes (any integer dtype) to fp64."""
    return _TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def encode_bruteforce(y) -> np.ndarray:
    """Encode fp32 values by searching the nearest of the 127 finite
    non-negative codes; a tie goes to the even code (even mantissa).

    Slow but transparent: compares |y| against every representable value.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    mags = _TABLE[:127]  # codes 0x00..0x7E, increasing
    for idx, v in enumerate(flat):
        sign = 0x80 if np.signbit(v) else 0x00
        if np.isnan(v):
            out[idx] = 0x7F | sign
            continue
        a = abs(v)
        if a >= MAX_FINITE:
            out[idx] = 0x7E | sign
            continue
        dist = np.abs(mags - a)
        best = dist.min()
        cands = np.nonzero(dist == best)[0]
        if len(cands) == 1:
            code = int(cands[0])
        else:  # exactly halfway between two neighbours
            evens = [int(c) for c in cands if (int(c) & 1) == 0]
            assert len(evens) == 1
            code = evens[0]
        out[idx] = code | sign
    return out.reshape(y.shape)


def encode_closed_form(y) -> np.ndarray:
    """Encode fp32 values by exponent/mantissa arithmetic (vectorised).

    For |y| in the normal range the spacing of codes is 2^(E-3) with
    E = floor(log2 |y|); in the subnormal range it is 2^-9.  |y| is divided
    by the spacing (exact in fp64), rounded half-to-even with ``np.rint``,
    multiplied back, and the resulting value is turned into bits.  A
    round-up that reaches the next binade is handled by recomputing the
    fields from the rounded value.
    """
    y = np.asarray(y, dtype=np.float32)
    v = y.astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    a = np.abs(v)
    nan = np.isnan(v)
    a_safe = np.where(nan, 0.0, a)
    sat = a_safe >= MAX_FINITE

    # spacing of representable values around a
    _, exp2 = np.frexp(np.where(a_safe > 0, a_safe, 1.0))  # a = f * 2^exp2, f in [0.5,1)
    E = exp2 - 1                                          # a in [2^E, 2^(E+1))
    normal = a_safe >= 2.0 ** -6
    quantum = np.where(normal, np.ldexp(1.0, E - 3), MIN_SUBNORMAL)
    r = np.rint(a_safe / quantum) * quantum               # rounded magnitude, exact
    r = np.minimum(r, MAX_FINITE)

    # fields of the rounded magnitude
    code = np.zeros(a.shape, dtype=np.int64)
    rn = r >= 2.0 ** -6
    _, er = np.frexp(np.where(rn, r, 1.0))
    Er = er - 1
    mant = np.where(rn, np.rint((r / np.ldexp(1.0, Er) - 1.0) * 8.0), 0).astype(np.int64)
    code = np.where(rn, ((Er + 7) << 3) | mant, np.rint(r / MIN_SUBNORMAL).astype(np.int64))
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


encode = encode_closed_form
