"""Pins for the oracle's page-layout index functions: they are bijections,
and a handful of offsets worked out by hand from the layout definition
(tests/golden/layout_offsets.json) come out as stated."""

import json
import os

import numpy as np

from oracle import layout

GOLD = os.path.join(os.path.dirname(__file__), "golden", "layout_offsets.json")


def test_bijection_per_block():
    for f in (layout.k_offset, layout.v_offset):
        o, d = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
        offs = f(o, d).reshape(-1)
        assert offs.min() == 0 and offs.max() == 16383
        assert len(np.unique(offs)) == 16384


def test_bijection_over_pages_and_heads():
    for Hkv in (1, 2):
        seen = []
        for p in range(4):
            for h in range(Hkv):
                seen.append(layout.block_base(p, h, Hkv) + layout.K_IDX.reshape(-1))
        allo = np.concatenate(seen)
        assert len(np.unique(allo)) == 4 * Hkv * 16384 == allo.max() + 1
        sc = np.concatenate([layout.scale_index(p, h, np.arange(128), Hkv)
                             for p in range(4) for h in range(Hkv)])
        assert len(np.unique(sc)) == 4 * Hkv * 128 == sc.max() + 1


def test_hand_worked_offsets():
    with open(GOLD) as f:
        g = json.load(f)
    for o, d, want in g["k"]:
        assert int(layout.k_offset(o, d)) == want, ("k", o, d)
    for o, d, want in g["v"]:
        assert int(layout.v_offset(o, d)) == want, ("v", o, d)


def test_chunks_are_contiguous_4k_runs():
    """Each 32-token chunk of a block occupies exactly one 4 KiB run."""
    for idx in (layout.K_IDX, layout.V_IDX):
        for c in range(4):
            run = idx[32 * c:32 * (c + 1)].reshape(-1)
            assert run.min() == 4096 * c and run.max() == 4096 * c + 4095


def test_sixteen_byte_pieces():
    """K: each aligned 16-byte piece holds 16 dims of one token (two runs of 8
    consecutive dims 32 apart).  V: each piece holds one dim of 8 tokens for
    two dims 16 apart."""
    inv_k = np.empty(16384, dtype=np.int64)
    inv_k[layout.K_IDX.reshape(-1)] = np.arange(16384)
    for piece in range(0, 16384, 16):
        tok = inv_k[piece:piece + 16] // 128
        dim = inv_k[piece:piece + 16] % 128
        assert len(set(tok.tolist())) == 1
        assert np.array_equal(np.diff(dim[:8]), np.ones(7)) and dim[8] - dim[0] == 32
    inv_v = np.empty(16384, dtype=np.int64)
    inv_v[layout.V_IDX.reshape(-1)] = np.arange(16384)
    for piece in range(0, 16384, 16):
        tok = inv_v[piece:piece + 16] // 128
        dim = inv_v[piece:piece + 16] % 128
        assert len(set(dim[:8].tolist())) == 1 and dim[8] == dim[0] + 16
        assert np.array_equal(tok[:8], tok[8:])
