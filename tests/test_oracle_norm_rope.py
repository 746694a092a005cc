"""Pins for the oracle of the fused norm + rotary writer (oracle/norm_rope):
closed forms of the rotation (zero angle, quarter turn), its invariants
(pair norms, composition, the two pair layouts related by a permutation),
the RMS norm's (unit RMS, scale invariance, the Gemma offset), loop-only
brute force, and the fp32 reading checked step by step against exact
rational arithmetic -- so a dropped term, a wrong sign, a swapped pair or a
changed summation order fails here."""

import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from exact_rational import round_f32, sqrt_f32
from oracle import bf16, layout, norm_rope as nr, writer

F = Fraction


def _x(T=5, H=None, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    shape = (T, 128) if H is None else (T, H, 128)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _tables(max_pos, rot, angles=None):
    if angles is None:
        return wl.rope_tables(max_pos, rot)
    return (np.cos(angles).astype(np.float32), np.sin(angles).astype(np.float32))


@pytest.mark.parametrize("rot", [128, 64, 4])
@pytest.mark.parametrize("neox", [True, False])
def test_zero_angle_is_identity(rot, neox):
    x = _x()
    c = np.ones((3, rot // 2), np.float32)
    s = np.zeros((3, rot // 2), np.float32)
    pos = np.array([0, 1, 2, 1, 0])
    assert np.array_equal(nr.rope(x, pos, c, s, rot, neox), x.astype(np.float64))
    assert np.array_equal(nr.rope_f32(x, pos, c, s, rot, neox), x)


@pytest.mark.parametrize("neox", [True, False])
def test_quarter_turn(neox):
    """cos 0, sin 1: each pair (a, b) becomes (-b, a), exactly."""
    x = _x(H=2)
    rot = 64
    c = np.zeros((1, rot // 2), np.float32)
    s = np.ones((1, rot // 2), np.float32)
    pos = np.zeros(x.shape[0], np.int64)
    i0, i1, _ = nr.pair_index(rot, neox)
    for y in (nr.rope(x, pos, c, s, rot, neox), nr.rope_f32(x, pos, c, s, rot, neox)):
        assert np.array_equal(y[..., i0], -x[..., i1])
        assert np.array_equal(y[..., i1], x[..., i0])
        assert np.array_equal(y[..., rot:], x[..., rot:])


@pytest.mark.parametrize("neox", [True, False])
def test_rotation_preserves_pair_norms_and_composes(neox):
    rot = 128
    rng = np.random.default_rng(3)
    th1 = rng.uniform(-7, 7, size=(1, rot // 2))
    th2 = rng.uniform(-7, 7, size=(1, rot // 2))
    x = _x(T=4).astype(np.float64)
    pos = np.zeros(4, np.int64)
    c1, s1 = np.cos(th1), np.sin(th1)
    c2, s2 = np.cos(th2), np.sin(th2)
    y = nr.rope(x, pos, c1, s1, rot, neox)
    i0, i1, _ = nr.pair_index(rot, neox)
    assert np.allclose(np.hypot(y[:, i0], y[:, i1]), np.hypot(x[:, i0], x[:, i1]), rtol=1e-14, atol=0)
    z = nr.rope(y, pos, c2, s2, rot, neox)
    direct = nr.rope(x, pos, np.cos(th1 + th2), np.sin(th1 + th2), rot, neox)
    assert np.allclose(z, direct, rtol=0, atol=1e-12)


def test_layouts_related_by_permutation():
    """Interleaved pairs on x equal rotate-halves pairs on x with its dims
    permuted (2i -> i, 2i+1 -> i + rot/2), permuted back."""
    rot = 96
    x = _x(T=6, H=3)
    c, s = _tables(50, rot)
    pos = np.array([0, 3, 49, 7, 7, 20])
    perm = np.arange(128)
    perm[:rot] = np.concatenate([np.arange(0, rot, 2), np.arange(1, rot, 2)])  # neox slot -> source dim
    xp = x[..., perm]
    yn = nr.rope(xp, pos, c, s, rot, True)
    back = np.empty_like(yn)
    back[..., perm] = yn
    yi = nr.rope(x, pos, c, s, rot, False)
    assert np.allclose(back, yi, rtol=0, atol=1e-15)


@pytest.mark.parametrize("neox", [True, False])
def test_bruteforce_loops(neox):
    rot, eps, off = 64, 1e-5, 1.0
    x = _x(T=3, H=2, seed=5)
    w = _x(T=1, seed=6)[0] * 0.1
    c, s = _tables(40, rot)
    pos = np.array([1, 17, 39])
    got = nr.norm_rope(x, pos, c, s, rot, neox, w, eps, off)
    for t in range(3):
        for h in range(2):
            row = [float(v) for v in x[t, h]]
            ms = math.fsum(v * v for v in row) / 128
            y = [row[d] / math.sqrt(ms + eps) * (off + float(w[d])) for d in range(128)]
            out = list(y)
            for i in range(rot // 2):
                a_i, b_i = (i, i + rot // 2) if neox else (2 * i, 2 * i + 1)
                ci, si = float(c[pos[t], i]), float(s[pos[t], i])
                out[a_i] = y[a_i] * ci - y[b_i] * si
                out[b_i] = y[b_i] * ci + y[a_i] * si
            assert np.allclose(got[t, h], out, rtol=1e-13, atol=1e-13)


def test_norm_closed_forms():
    x = _x(T=8, seed=7, scale=3.0)
    y = nr.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    # Gemma form with zero weight equals the plain form with unit weight
    assert np.array_equal(nr.rms_norm(x, np.zeros(128), 0.0, 1.0), y)
    # scale invariance without eps; the weight scales each dim
    assert np.allclose(nr.rms_norm(x * np.float32(1024.0), np.ones(128), 0.0), y, rtol=1e-13)
    w = np.linspace(-2, 2, 128)
    assert np.allclose(nr.rms_norm(x, w, 0.0), y * w, rtol=1e-14)


def test_tree_sum_order():
    v = np.array([1e8, 1.0, -1e8, 1.0, 3.0, 2.0 ** -30, 5.0, 7.0], np.float32)
    # by hand: ((v0+v1)+(v2+v3)) + ((v4+v5)+(v6+v7)), each rounded to fp32
    f = np.float32
    want = f(f(f(v[0] + v[1]) + f(v[2] + v[3])) + f(f(v[4] + v[5]) + f(v[6] + v[7])))
    assert nr.tree_sum_f32(v) == want
    assert want == f(15.0)
    seq = f(0.0)
    for t in v:
        seq = f(seq + t)
    assert seq == f(16.0)    # a left-to-right sum gives another value
    ints = np.arange(128, dtype=np.float32)
    assert nr.tree_sum_f32(ints) == 127 * 128 / 2
    rng = np.random.default_rng(9)
    r = rng.standard_normal(128).astype(np.float32)
    err = abs(float(nr.tree_sum_f32(r)) - math.fsum(float(t) for t in r))
    assert err <= 7 * 2.0 ** -24 * math.fsum(abs(float(t)) for t in r)


def _exact_row(x, w, eps, off, pos, c, s, rot, neox):
    """The fp32 reading of one row evaluated with exact rationals, rounding
    after every operation as the reading states."""
    X = [F(float(t)) for t in x]
    if w is not None:
        sq = [round_f32(t * t) for t in X]
        while len(sq) > 1:
            sq = [round_f32(sq[i] + sq[i + 1]) for i in range(0, len(sq), 2)]
        m = round_f32(sq[0] / 128)
        v = round_f32(m + F(float(np.float32(eps))))
        inv = round_f32(1 / sqrt_f32(v))
        X = [round_f32(round_f32(X[d] * inv) * round_f32(F(float(np.float32(off))) + F(float(w[d]))))
             for d in range(128)]
    Y = list(X)
    for i in range(rot // 2):
        a_i, b_i = (i, i + rot // 2) if neox else (2 * i, 2 * i + 1)
        ci, si = F(float(c[pos, i])), F(float(s[pos, i]))
        Y[a_i] = round_f32(round_f32(X[a_i] * ci) - round_f32(X[b_i] * si))
        Y[b_i] = round_f32(round_f32(X[b_i] * ci) + round_f32(X[a_i] * si))
    return Y


@pytest.mark.parametrize("neox,off,rot", [(True, 1.0, 128), (False, 0.0, 64), (True, 0.0, 0)])
def test_f32_reading_is_stepwise_ieee(neox, off, rot):
    x = _x(T=3, seed=11, scale=2.0)
    x[2] *= np.float32(1e-20)   # tiny row: eps dominates
    w = _x(T=1, seed=12)[0] * np.float32(0.3)
    c, s = _tables(64, max(rot, 4))
    pos = np.array([5, 63, 0])
    eps = 1e-6
    got = nr.norm_rope_f32(x, pos, c, s, rot, neox, w, eps, off)
    for t in range(3):
        want = _exact_row(x[t], w, eps, off, pos[t], c, s, rot, neox)
        assert [F(float(g)) for g in got[t]] == want, t


def test_f32_reading_close_to_textbook():
    x = _x(T=16, H=2, seed=13, scale=4.0)
    w = _x(T=1, seed=14)[0] * 0.5
    c, s = _tables(100, 128)
    pos = np.arange(16) * 6
    a = nr.norm_rope_f32(x, pos, c, s, 128, True, w, 1e-6, 1.0).astype(np.float64)
    b = nr.norm_rope(x, pos, c.astype(np.float64), s.astype(np.float64), 128, True, w, 1e-6, 1.0)
    assert np.max(np.abs(a - b)) <= 2.0 ** -19 * np.max(np.abs(b))


def test_fused_write_goes_through_the_one_writer():
    T, Hkv, nb = 9, 2, 2
    rng = np.random.default_rng(15)
    k = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    q = rng.standard_normal((T, 16 * Hkv, 128)).astype(np.float32)
    slots = rng.permutation(nb * 128)[:T].astype(np.int64)
    pos = rng.integers(0, 300, size=T)
    c, s = _tables(256, 64)
    kw, qw = _x(T=1, seed=16)[0], _x(T=1, seed=17)[0]
    fresh = lambda: (np.zeros(nb * Hkv * 16384, np.uint8), np.zeros(nb * Hkv * 16384, np.uint8),
                     np.zeros(nb * Hkv * 128, np.float32), np.zeros(nb * Hkv * 128, np.float32))
    # no norm, no rotation: exactly kv_quant_write's output; q passes as bf16
    a = fresh()
    qa = nr.norm_rope_write_ref(k, v, slots, pos, c, s, 0, True, None, 1e-6, 0.0, *a, writer.PER_TOKEN, Hkv, q=q)
    b = fresh()
    writer.quant_write_ref(k, v, slots, *b, writer.PER_TOKEN, Hkv)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert np.array_equal(qa, bf16.encode(q))
    # with both: the writer on the transformed K (positions clamped to the table)
    a = fresh()
    qa = nr.norm_rope_write_ref(k, v, slots, pos, c, s, 64, False, kw, 1e-6, 1.0, *a, writer.PER_TOKEN, Hkv,
                                q=q, q_weight=qw)
    pc = np.minimum(pos, 255)
    b = fresh()
    writer.quant_write_ref(nr.norm_rope_f32(k, pc, c, s, 64, False, kw, 1e-6, 1.0), v, slots, *b,
                           writer.PER_TOKEN, Hkv)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert np.array_equal(qa, bf16.encode(nr.norm_rope_f32(q, pc, c, s, 64, False, qw, 1e-6, 1.0)))
    # V is stored as it comes
    o = int(slots[0]) % 128
    base = int(layout.block_base(int(slots[0]) // 128, 0, Hkv))
    vb = fresh()
    writer.quant_write_ref(k, v, slots, *vb, writer.PER_TOKEN, Hkv)
    assert np.array_equal(a[1][base + layout.v_offset(o, np.arange(128))],
                          vb[1][base + layout.v_offset(o, np.arange(128))])
