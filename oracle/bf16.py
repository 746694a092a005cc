"""bfloat16 as the unquantized KV element: 1 sign, 8 exponent, 7 mantissa
bits, the top half of an IEEE fp32.

Test infrastructure only (see ``oracle/__init__``).

Decoding is exact (the 16 bits shifted into the top of an fp32).  Encoding
from fp32 rounds to nearest, ties to even, on the dropped 16 bits; NaN stays
NaN (quiet, sign kept).  The pages keep a BF16-KV control next to the FP8
cache (ROCm/ATOM pull request 2710, "Test Result": FP8 and BF16 KV rows;
pull request 2614's follow-up: the BF16-KV baseline).
"""

import numpy as np


def decode(bits) -> np.ndarray:
    """fp64 values of bf16 bit patterns (uint16)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def encode(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    quiet = (u >> 16) | 0x40
    return np.where(nan, quiet, rounded).astype(np.uint16)
