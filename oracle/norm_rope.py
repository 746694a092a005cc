"""Reference for the cache writer fused with the key norm and rotary embedding.

Test infrastructure only (see ``oracle/__init__``).

What the pages say: a serving stack writes K/V into the FP8 cache from two
places -- after rotary position embedding alone, and after a Gemma-style
norm followed by the rotary embedding -- and the two cache-write branches
drifted apart; the review asks for one shared writer (ROCm/ATOM pull request
2710 review, "Smaller": ``_gemma_norm_rope_then_cache`` repeats the FP8 /
non-FP8 branch of ``rope_cache``).  Its "Changes" section fuses the query /
key norm, the rotary embedding and the cache write for prefill steps.  The
pages give neither the norm's nor the rotary embedding's parameters, so they
are all the caller's: a per-dimension norm weight and epsilon (with the
Gemma convention of scaling by 1 + weight as an option), cosine and sine
tables indexed by position, the rotary width and the pair layout.

The textbook definitions, in fp64 (``rms_norm``, ``rope``, ``norm_rope``):

* RMS norm over the 128 dims of one head: y_d = x_d / sqrt(mean_e(x_e^2) +
  eps) * (offset + w_d), offset 0 (plain) or 1 (Gemma).
* Rotary embedding over the first ``rot`` dims (the rest pass unchanged):
  pairs (i, i + rot/2) ("neox", rotate halves) or (2i, 2i + 1)
  (interleaved), i < rot/2; with c = cos[pos, i], s = sin[pos, i] the pair
  (a, b) becomes (a c - b s, b c + a s) -- a rotation by the table's angle.
* K goes through the norm with the key weight, then the rotary embedding,
  then the one cache writer (``writer.quant_write_ref``); V is written as
  it comes; a query, if given, gets the same norm (its own weight) and
  rotary embedding and is returned as bf16.

The fp32 reading (``norm_rope_f32``), which the library's kernel follows
operation for operation, so that cache bytes and scales can be compared bit
for bit: every step is one IEEE fp32 operation rounded to nearest even, with
no fused multiply-add:

1. sq_d = x_d * x_d;
2. S = sum of sq over d as a balanced binary tree in dimension order (sq_0
   + sq_1, sq_2 + sq_3, ... then adjacent pairs of those, ...);
3. m = S / 128 (exact); v = m + eps; r = sqrt(v); inv = 1 / r;
4. y_d = (x_d * inv) * (offset + w_d);
5. rotated pair: (a*c - b*s, b*c + a*s), each product rounded, then the
   difference or sum rounded.
"""

import numpy as np

from . import bf16, writer

DIM = 128


def _check_rot(rot):
    if rot < 0 or rot > DIM or rot % 4 != 0:
        raise ValueError("rotary width must be a multiple of 4 in [0, 128]")


def pair_index(rot: int, neox: bool):
    """(first, second) dims of the rotary pairs, and the table column i of
    each pair."""
    _check_rot(rot)
    half = rot // 2
    i = np.arange(half)
    if neox:
        return i, i + half, i
    return 2 * i, 2 * i + 1, i


# ---- textbook definitions, fp64 ----------------------------------------

def rms_norm(x, w, eps: float, offset: float = 0.0) -> np.ndarray:
    """fp64 RMS norm over the last axis (128 dims)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * (float(offset) + w)


def rope(x, pos, cos, sin, rot: int, neox: bool) -> np.ndarray:
    """fp64 rotary embedding of x [..., T, (H,) 128] at positions pos [T]
    with tables cos, sin [max_pos, rot/2] (used as given)."""
    x = np.array(x, dtype=np.float64)
    if rot == 0:
        return x
    i0, i1, ci = pair_index(rot, neox)
    pos = np.asarray(pos, dtype=np.int64)
    c = np.asarray(cos, dtype=np.float64)[pos][:, ci]          # [T, rot/2]
    s = np.asarray(sin, dtype=np.float64)[pos][:, ci]
    if x.ndim == 3:
        c, s = c[:, None, :], s[:, None, :]
    a, b = x[..., i0].copy(), x[..., i1].copy()
    x[..., i0] = a * c - b * s
    x[..., i1] = b * c + a * s
    return x


def norm_rope(x, pos, cos, sin, rot, neox, w=None, eps=1e-6, offset=0.0) -> np.ndarray:
    """fp64: the norm (if a weight is given), then the rotary embedding."""
    y = np.asarray(x, dtype=np.float64)
    if w is not None:
        y = rms_norm(y, w, eps, offset)
    return rope(y, pos, cos, sin, rot, neox)


# ---- the fp32 reading ---------------------------------------------------

def tree_sum_f32(v) -> np.ndarray:
    """fp32 sum over the last axis (a power of two long) as a balanced
    binary tree in index order, every addition rounded to fp32."""
    s = np.asarray(v, dtype=np.float32)
    while s.shape[-1] > 1:
        s = (s[..., 0::2] + s[..., 1::2]).astype(np.float32)
    return s[..., 0]


def rms_norm_f32(x, w, eps: float, offset: float = 0.0) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    sq = (x * x).astype(np.float32)
    S = tree_sum_f32(sq)
    m = (S / np.float32(DIM)).astype(np.float32)
    v = (m + np.float32(eps)).astype(np.float32)
    r = np.sqrt(v).astype(np.float32)
    inv = (np.float32(1.0) / r).astype(np.float32)
    wp = (np.float32(offset) + np.asarray(w, dtype=np.float32)).astype(np.float32)
    return ((x * inv[..., None]).astype(np.float32) * wp).astype(np.float32)


def rope_f32(x, pos, cos, sin, rot: int, neox: bool) -> np.ndarray:
    x = np.array(x, dtype=np.float32)
    if rot == 0:
        return x
    i0, i1, ci = pair_index(rot, neox)
    pos = np.asarray(pos, dtype=np.int64)
    c = np.asarray(cos, dtype=np.float32)[pos][:, ci]
    s = np.asarray(sin, dtype=np.float32)[pos][:, ci]
    if x.ndim == 3:
        c, s = c[:, None, :], s[:, None, :]
    a, b = x[..., i0].copy(), x[..., i1].copy()
    ac, bs = (a * c).astype(np.float32), (b * s).astype(np.float32)
    bc, as_ = (b * c).astype(np.float32), (a * s).astype(np.float32)
    x[..., i0] = (ac - bs).astype(np.float32)
    x[..., i1] = (bc + as_).astype(np.float32)
    return x


def norm_rope_f32(x, pos, cos, sin, rot, neox, w=None, eps=1e-6, offset=0.0) -> np.ndarray:
    """The fp32 reading of ``norm_rope`` (see the module text)."""
    y = np.asarray(x, dtype=np.float32)
    if w is not None:
        y = rms_norm_f32(y, w, eps, offset)
    return rope_f32(y, pos, cos, sin, rot, neox)


def norm_rope_write_ref(k_new, v_new, slot_mapping, positions, cos, sin, rot, neox,
                        k_weight, eps, offset, k_cache, v_cache, k_scale, v_scale, mode,
                        num_kv_heads, q=None, q_weight=None, kv_dtype="fp8"):
    """The fused writer: K through the key norm (if ``k_weight`` is not
    None) and the rotary embedding in the fp32 reading, then the one cache
    writer with V as it comes.  Returns the query's bf16 bit patterns
    [T, Hq, 128] (uint16) after its norm and rotary embedding, or None.
    Positions are clamped into the tables' range, as the kernel reads
    them."""
    k_new = np.asarray(k_new, dtype=np.float32)
    max_pos = np.asarray(cos).shape[0]
    pos = np.clip(np.asarray(positions, dtype=np.int64), 0, max_pos - 1)
    k_t = norm_rope_f32(k_new, pos, cos, sin, rot, neox, k_weight, eps, offset)
    if kv_dtype == "bf16":
        writer.write_bf16_ref(k_t, v_new, slot_mapping, k_cache, v_cache, num_kv_heads)
    else:
        writer.quant_write_ref(k_t, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, mode,
                               num_kv_heads)
    if q is None:
        return None
    q_t = norm_rope_f32(np.asarray(q, dtype=np.float32), pos, cos, sin, rot, neox, q_weight, eps, offset)
    return bf16.encode(q_t)
