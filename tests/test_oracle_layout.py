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


# ---- BF16 pages (element offsets) -------------------------------------------

def test_bf16_bijection_per_block():
    for idx in (layout.K_IDX_BF16, layout.V_IDX_BF16):
        offs = idx.reshape(-1)
        assert offs.min() == 0 and offs.max() == 16383
        assert len(np.unique(offs)) == 16384


def test_bf16_hand_worked_offsets():
    with open(GOLD) as f:
        g = json.load(f)
    for o, d, want in g["k_bf16"]:
        assert int(layout.k_offset_bf16(o, d)) == want, ("k", o, d)
    for o, d, want in g["v_bf16"]:
        assert int(layout.v_offset_bf16(o, d)) == want, ("v", o, d)


def test_bf16_chunks_are_contiguous_8k_runs():
    """Each 32-token chunk of a bf16 block is one run of 4096 elements."""
    for idx in (layout.K_IDX_BF16, layout.V_IDX_BF16):
        for c in range(4):
            run = idx[32 * c:32 * (c + 1)].reshape(-1)
            assert run.min() == 4096 * c and run.max() == 4096 * c + 4095


def test_bf16_eight_element_pieces():
    """K: each aligned 8-element piece is 8 consecutive dims of one token,
    and the pieces of one 512-element row are tokens r (16 of them) for the
    four 8-dim groups of one 32-dim k-step.  V: each piece is one dim of 8
    tokens, slot e -> token 16*(e//4) + 4*g + e%4 of the chunk."""
    inv_k = np.empty(16384, dtype=np.int64)
    inv_k[layout.K_IDX_BF16.reshape(-1)] = np.arange(16384)
    for piece in range(0, 16384, 8):
        tok = inv_k[piece:piece + 8] // 128
        dim = inv_k[piece:piece + 8] % 128
        assert len(set(tok.tolist())) == 1
        assert np.array_equal(np.diff(dim), np.ones(7)) and dim[0] % 8 == 0
        row, lane = divmod(piece % 4096, 512)
        lane //= 8
        assert tok[0] % 16 == lane % 16 and (dim[0] % 32) // 8 == lane // 16
        assert dim[0] // 32 == row % 4 and (tok[0] % 32) // 16 == row // 4
    inv_v = np.empty(16384, dtype=np.int64)
    inv_v[layout.V_IDX_BF16.reshape(-1)] = np.arange(16384)
    for piece in range(0, 16384, 8):
        tok = inv_v[piece:piece + 8] // 128
        dim = inv_v[piece:piece + 8] % 128
        assert len(set(dim.tolist())) == 1
        row, lane = divmod(piece % 4096, 512)
        lane //= 8
        assert dim[0] == 16 * row + lane % 16
        g = lane // 16
        want = [32 * (piece // 4096) + 16 * (e // 4) + 4 * g + e % 4 for e in range(8)]
        assert tok.tolist() == want
