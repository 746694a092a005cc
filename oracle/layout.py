"""Byte layout of the page-shuffled FP8 KV cache and its scale arrays.

Test infrastructure only (see ``oracle/__init__``).

The pages say the cache is "page-shuffled" FP8 with per-token K/V scales and
that K bytes, V bytes and both scales are viewed per KV head in one
consistent way (ROCm/ATOM pull request 2614, sections Problem and Change),
but never give the byte order.  The order below is this library's own
definition; the oracle follows it through these index functions, written
from the definition, and shares nothing with the GPU code.

A page holds 128 tokens.  For physical page ``p`` and KV head ``h`` (of
``Hkv``) there is one 16384-byte K block and one 16384-byte V block at byte
``(p * Hkv + h) * 16384`` of the K and V cache arrays, and 128 fp32 scales
at element ``(p * Hkv + h) * 128 + o`` of each scale array (``o`` = token
slot in the page).  Inside a block, token slot ``o`` in [0, 128) and head
dimension ``d`` in [0, 128) sit at

K: ``c = o // 32, tau = (o % 32) // 16, r = o % 16``;
   ``j = d // 32, g = (d % 32) // 8, u = d % 8``;
   offset ``= 4096*c + 1024*(2*tau + j//2) + 16*(16*g + r) + 8*(j % 2) + u``.

V: ``c = o // 32, tau = (o % 32) // 16, w = o % 16``;
   ``g = w // 4, e = 4*tau + w % 4``; ``delta = d // 16, r = d % 16``;
   offset ``= 4096*c + 1024*(delta // 2) + 16*(16*g + r) + 8*(delta % 2) + e``.

Every 32-token chunk ``c`` is one contiguous 4 KiB run of each block; within
it, 1 KiB row ``i`` is read as 64 consecutive 16-byte pieces.

BF16 pages (the unquantized cache; same principle, 2-byte elements): a
(page, head) block is 16384 bf16 elements (32 KiB) at element
``(p * Hkv + h) * 16384``, and inside it

K: ``c, tau, r, j, g, u`` as above;
   element ``= 4096*c + 512*(4*tau + j) + 8*(16*g + r) + u``.

V: ``c, tau, w, g, e, delta, r`` as above;
   element ``= 4096*c + 512*delta + 8*(16*g + r) + e``.

so each 32-token chunk is one contiguous 8 KiB run and every aligned
16-byte piece is 8 elements of one lane's operand.
"""

import numpy as np

PAGE = 128
DIM = 128
BLOCK_BYTES = PAGE * DIM


def k_offset(o, d):
    """Byte offset of K[token slot o, dim d] inside one (page, head) block."""
    o = np.asarray(o, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    c = o // 32
    tau = (o % 32) // 16
    r = o % 16
    j = d // 32
    g = (d % 32) // 8
    u = d % 8
    return 4096 * c + 1024 * (2 * tau + j // 2) + 16 * (16 * g + r) + 8 * (j % 2) + u


def v_offset(o, d):
    """Byte offset of V[token slot o, dim d] inside one (page, head) block."""
    o = np.asarray(o, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    c = o // 32
    tau = (o % 32) // 16
    w = o % 16
    g = w // 4
    e = 4 * tau + w % 4
    delta = d // 16
    r = d % 16
    return 4096 * c + 1024 * (delta // 2) + 16 * (16 * g + r) + 8 * (delta % 2) + e


def k_offset_bf16(o, d):
    """Element offset of K[token slot o, dim d] in one bf16 (page, head) block."""
    o = np.asarray(o, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    c = o // 32
    tau = (o % 32) // 16
    r = o % 16
    j = d // 32
    g = (d % 32) // 8
    u = d % 8
    return 4096 * c + 512 * (4 * tau + j) + 8 * (16 * g + r) + u


def v_offset_bf16(o, d):
    """Element offset of V[token slot o, dim d] in one bf16 (page, head) block."""
    o = np.asarray(o, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    c = o // 32
    tau = (o % 32) // 16
    w = o % 16
    g = w // 4
    e = 4 * tau + w % 4
    delta = d // 16
    r = d % 16
    return 4096 * c + 512 * delta + 8 * (16 * g + r) + e


def block_base(page, head, num_kv_heads):
    """Byte offset of the (page, head) block in a K or V cache array."""
    return (np.asarray(page, dtype=np.int64) * num_kv_heads + head) * BLOCK_BYTES


def scale_index(page, head, slot, num_kv_heads):
    """Element index of the per-token scale of (page, head, token slot)."""
    return (np.asarray(page, dtype=np.int64) * num_kv_heads + head) * PAGE + slot


# Index grids for a whole block: K_IDX[o, d] = k_offset(o, d), same for V.
_O, _D = np.meshgrid(np.arange(PAGE), np.arange(DIM), indexing="ij")
K_IDX = k_offset(_O, _D)
V_IDX = v_offset(_O, _D)
K_IDX_BF16 = k_offset_bf16(_O, _D)
V_IDX_BF16 = v_offset_bf16(_O, _D)


def gather_block(cache_flat: np.ndarray, page: int, head: int, num_kv_heads: int, kind: str) -> np.ndarray:
    """Codes of one (page, head) block as a [128 tokens, 128 dims] uint8 array."""
    base = int(block_base(page, head, num_kv_heads))
    idx = K_IDX if kind == "k" else V_IDX
    return cache_flat[base + idx]
