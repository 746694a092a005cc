"""Reference cache writer: quantize new K/V rows to e4m3 and store them.

Test infrastructure only (see ``oracle/__init__``).

What it follows:

* Per-token scales: one fp32 scale for every (token, KV head), for K and for
  V separately (ROCm/ATOM pull request 2614, section Problem; vLLM pull
  request 52060, "Suggested Fix" names the per-token/head mode).  The scale
  is amax / 448, 448 being the largest e4m3fn magnitude (the workload
  definition that quantizes K/V "with a per-token per-head fp32 scale =
  amax/448").
* Scalar mode (vLLM pull request 52060, "Suggested Fix", KV_SCALE_MODE 1):
  one caller-given fp32 scale for all of K and one for all of V.
* No-scale mode: the values are encoded as they are (scale 1).
* One writer for every path (ROCm/ATOM pull request 2710 review, "Smaller":
  two copies of the FP8 cache-write branch drifted apart).

Readings where the pages are silent (each listed in the design notes):
two roundings, fp32 division first and then round-to-nearest-even into
e4m3; saturation at 448; an all-zero row stores scale 0 and sign-only codes;
a negative slot means "skip this token"; a slot beyond the cache is skipped
too.
"""

import numpy as np

from . import bf16, e4m3, layout

NONE, SCALAR, PER_TOKEN = 0, 1, 2
E4M3_MAX = np.float32(448.0)


def quantize_rows(x: np.ndarray, mode: int, scalar_scale=None):
    """Quantize rows of 128 values.

    x: float32 [..., 128].  Returns (codes uint8 [..., 128], scale float32
    [...]) where ``scale`` is what is stored for per-token mode (for the
    other modes it is the scale that was used).
    """
    x = np.asarray(x, dtype=np.float32)
    if mode == PER_TOKEN:
        amax = np.max(np.abs(x), axis=-1)                      # exact in fp32
        scale = (amax / E4M3_MAX).astype(np.float32)           # fp32 IEEE division
        zero = scale == 0
        safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
        y = (x / safe[..., None]).astype(np.float32)           # fp32 IEEE division
        y = np.where(zero[..., None], x, y)                    # all-zero row: keep signed zeros
    elif mode == SCALAR:
        s = np.float32(scalar_scale)
        y = (x / s).astype(np.float32)
        scale = np.full(x.shape[:-1], s, dtype=np.float32)
    elif mode == NONE:
        y = x
        scale = np.ones(x.shape[:-1], dtype=np.float32)
    else:
        raise ValueError(f"unknown scale mode {mode}")
    return e4m3.encode(y), scale


def quant_write_ref(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                    mode: int, num_kv_heads: int):
    """Write T new tokens into the cache arrays (in place).

    k_new, v_new: float32 [T, Hkv, 128] (bf16 inputs are passed widened,
    which is exact).  slot_mapping: int64 [T]; slot = page * 128 + token
    slot.  k_cache, v_cache: flat uint8 arrays of num_blocks * Hkv * 16384
    bytes.  k_scale, v_scale: flat float32 arrays of num_blocks * Hkv * 128
    (per-token mode: written), or 1-element arrays holding the scalar scale
    (scalar mode: read), or None (no-scale mode).
    """
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    T, Hkv, D = k_new.shape
    assert Hkv == num_kv_heads and D == layout.DIM
    num_blocks = k_cache.size // (Hkv * layout.BLOCK_BYTES)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = (slots >= 0) & (slots < num_blocks * layout.PAGE)
    ts = np.nonzero(keep)[0]
    if len(ts) == 0:
        return
    pages = slots[ts] // layout.PAGE
    offs = slots[ts] % layout.PAGE

    ks_in = None if mode != SCALAR else np.float32(np.asarray(k_scale).reshape(-1)[0])
    vs_in = None if mode != SCALAR else np.float32(np.asarray(v_scale).reshape(-1)[0])
    kc, ksc = quantize_rows(k_new[ts], mode, ks_in)            # [n, Hkv, 128], [n, Hkv]
    vc, vsc = quantize_rows(v_new[ts], mode, vs_in)

    heads = np.arange(Hkv)
    base = layout.block_base(pages[:, None], heads[None, :], Hkv)          # [n, Hkv]
    dims = np.arange(layout.DIM)
    kidx = base[:, :, None] + layout.k_offset(offs[:, None, None], dims[None, None, :])
    vidx = base[:, :, None] + layout.v_offset(offs[:, None, None], dims[None, None, :])
    k_cache[kidx] = kc
    v_cache[vidx] = vc
    if mode == PER_TOKEN:
        sidx = layout.scale_index(pages[:, None], heads[None, :], offs[:, None], Hkv)
        k_scale[sidx] = ksc
        v_scale[sidx] = vsc


def write_bf16_ref(k_new, v_new, slot_mapping, k_cache, v_cache, num_kv_heads: int):
    """The same writer for the unquantized BF16 cache: each value is stored
    as bf16 (round to nearest even from fp32; bf16 inputs, passed widened,
    are stored unchanged) at the bf16 layout's element offset.  k_cache,
    v_cache: flat uint16 arrays of num_blocks * Hkv * 16384 elements."""
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    T, Hkv, D = k_new.shape
    assert Hkv == num_kv_heads and D == layout.DIM
    num_blocks = k_cache.size // (Hkv * layout.BLOCK_BYTES)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = (slots >= 0) & (slots < num_blocks * layout.PAGE)
    ts = np.nonzero(keep)[0]
    if len(ts) == 0:
        return
    pages = slots[ts] // layout.PAGE
    offs = slots[ts] % layout.PAGE
    heads = np.arange(Hkv)
    base = (pages[:, None] * Hkv + heads[None, :]) * layout.BLOCK_BYTES
    dims = np.arange(layout.DIM)
    kidx = base[:, :, None] + layout.k_offset_bf16(offs[:, None, None], dims[None, None, :])
    vidx = base[:, :, None] + layout.v_offset_bf16(offs[:, None, None], dims[None, None, :])
    k_cache[kidx] = bf16.encode(k_new[ts])
    v_cache[vidx] = bf16.encode(v_new[ts])
