"""The length-balanced partition layout computes max(1, ceil(pages / p)) per
request as a float quotient (operands exact below 2^24, times the hardware
reciprocal) corrected once each way.  This emulates that arithmetic in
float32 on the host, with the reciprocal perturbed by up to 2 ulp either
way, and checks it against exact integer division over the kernel's input
range (pages <= 2^20 per request, any partition size p >= 1)."""

import numpy as np


def corrected_quotient(n, d, ulps):
    r = np.float32(1.0) / np.float32(d)
    for _ in range(abs(ulps)):
        r = np.nextafter(r, np.float32(np.inf) if ulps > 0 else np.float32(0.0))
    q = int(np.float32(np.float32(n) * r))  # truncation toward zero, as the float -> uint conversion
    rem = n - q * d
    if rem < 0:
        q -= 1
    elif rem >= d:
        q += 1
    return q


def test_corrected_float_quotient_is_exact_ceil():
    rng = np.random.default_rng(20260)
    edges = [0, 1, 2, 127, 128, 129, 2**20 - 1, 2**20]
    for i in range(40000):
        pages = int(rng.choice(edges)) if i % 4 == 0 else int(rng.integers(0, 2**20 + 1))
        p = int(rng.integers(1, 2**26)) if i % 3 == 0 else int(rng.integers(1, 4097))
        n = pages + p - 1
        want = n // p
        for u in (-2, -1, 0, 1, 2):
            assert corrected_quotient(n, p, u) == want, (pages, p, u)
    # a page count that is an exact multiple, with the quotient's float
    # product landing just below the integer
    for p in (3, 7, 11, 13, 127, 1000, 4095):
        for k in (1, 1000, 2**20 // p):
            assert corrected_quotient(k * p + p - 1, p, -2) == k
