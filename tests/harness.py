"""Test-side plumbing: put a workload on the GPU through the library's own
writer, build the oracle's side of the same workload, and compare.

The GPU side and the oracle side start from the same seeded inputs
(``workloads``); nothing the oracle uses comes from the GPU.
"""

import math

import numpy as np
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl
from oracle import attention as oatt
from oracle import layout as olay
from oracle import writer as owr

POISON_SCALE = 1e3


def poison_arrays(w, nb=None):
    """Initial cache contents: random finite e4m3 codes and scales of 1e3,
    so a read of anything the call should not touch shows in the output.
    A bf16 cache gets random 16-bit patterns, NaN and infinities included:
    a slot past the context that leaks into the output shows as non-finite."""
    nb = w.num_blocks if nb is None else nb
    rng = np.random.default_rng(w.seed + 99)
    if w.kv_dtype == "bf16":
        kc = rng.integers(0, 1 << 16, size=nb * w.Hkv * 16384, dtype=np.uint16)
        vc = rng.integers(0, 1 << 16, size=nb * w.Hkv * 16384, dtype=np.uint16)
        return kc, vc, None, None
    kc = rng.integers(0, 0x7F, size=nb * w.Hkv * 16384, dtype=np.uint8)
    vc = rng.integers(0, 0x7F, size=nb * w.Hkv * 16384, dtype=np.uint8)
    ks = np.full(nb * w.Hkv * 128, POISON_SCALE, dtype=np.float32)
    return kc, vc, ks, ks.copy()


class GpuCase:
    """A workload resident on the GPU, its cache written by kv_quant_write."""

    def __init__(self, w, device="cuda:0", kv_dtype=torch.uint8, in_dtype=torch.float32,
                 poison=True):
        self.w = w
        self.dev = torch.device(device)
        nb, Hkv = w.num_blocks, w.Hkv
        if w.kv_dtype == "bf16":
            # poison drawn on the device (a 128K-context bf16 cache is GiBs):
            # every 16-bit pattern, NaN and infinities included
            kv_dtype = torch.bfloat16
            self.kc = torch.zeros(nb, Hkv, 16384, dtype=torch.int16, device=self.dev)
            self.vc = torch.zeros_like(self.kc)
            if poison:
                g = torch.Generator(device=self.dev)
                g.manual_seed(w.seed + 99)
                for t in (self.kc, self.vc):
                    t.random_(-32768, 32768, generator=g)
            self.kc = self.kc.view(torch.bfloat16)
            self.vc = self.vc.view(torch.bfloat16)
            self.ks = self.vs = None
        elif poison:
            kc, vc, ks, vs = poison_arrays(w)
            self.kc = torch.from_numpy(kc).to(self.dev).view(nb, Hkv, 16384)
            self.vc = torch.from_numpy(vc).to(self.dev).view(nb, Hkv, 16384)
            self.ks = torch.from_numpy(ks).to(self.dev).view(nb, Hkv, 128)
            self.vs = torch.from_numpy(vs).to(self.dev).view(nb, Hkv, 128)
        else:
            self.kc = torch.zeros(nb, Hkv, 16384, dtype=torch.uint8, device=self.dev)
            self.vc = torch.zeros_like(self.kc)
            self.ks = torch.full((nb, Hkv, 128), POISON_SCALE, device=self.dev)
            self.vs = torch.full((nb, Hkv, 128), POISON_SCALE, device=self.dev)
        if kv_dtype == torch.float8_e4m3fn:
            self.kc = self.kc.view(torch.float8_e4m3fn)
            self.vc = self.vc.view(torch.float8_e4m3fn)
        self.mode = w.mode
        if w.mode == wl.SCALAR:
            self.ks_arg = torch.tensor([w.k_scalar], dtype=torch.float32, device=self.dev)
            self.vs_arg = torch.tensor([w.v_scalar], dtype=torch.float32, device=self.dev)
        elif w.mode == wl.NONE:
            self.ks_arg = self.vs_arg = None
        else:
            self.ks_arg, self.vs_arg = self.ks, self.vs
        self.in_dtype = in_dtype
        for b in range(w.B):
            self.write_request(b)
        self.q = torch.from_numpy(w.q).to(self.dev).to(torch.bfloat16)
        self.bt = torch.from_numpy(w.block_table).to(self.dev)
        self.ctx = torch.from_numpy(w.ctx).to(self.dev)
        self.cu = None if w.cu is None else torch.from_numpy(w.cu).to(self.dev)
        self.sp = None if w.sparse is None else torch.from_numpy(w.sparse).to(self.dev)
        self.out = torch.empty(w.rows, w.Hq, 128, dtype=torch.bfloat16, device=self.dev)

    def write_request(self, b, chunk_pages=256):
        pages = self.w.written[b]
        for i in range(0, len(pages), chunk_pages):
            k, v, s = self.w.request_kv(b, pages[i:i + chunk_pages])
            kt = torch.from_numpy(k).to(self.dev).to(self.in_dtype)
            vt = torch.from_numpy(v).to(self.dev).to(self.in_dtype)
            st = torch.from_numpy(s).to(self.dev)
            pa.kv_quant_write(kt, vt, st, self.kc, self.vc, self.ks_arg, self.vs_arg, self.mode)

    def decode(self, out=None, **kw):
        out = self.out if out is None else out
        if kw:
            pa.pa_decode_ex(self.q, self.kc, self.vc, self.ks_arg, self.vs_arg, self.bt, self.ctx,
                            self.cu, self.sp, self.mode, out, **kw)
        else:
            pa.pa_decode(self.q, self.kc, self.vc, self.ks_arg, self.vs_arg, self.bt, self.ctx,
                         self.cu, self.sp, self.mode, out)
        return out


def oracle_cache(w):
    """The oracle's cache for a (small) workload: poison, then every written
    page through the reference writer."""
    kc, vc, ks, vs = poison_arrays(w)
    if w.kv_dtype == "bf16":
        for b in range(w.B):
            k, v, s = w.request_kv(b)
            owr.write_bf16_ref(k, v, s, kc, vc, w.Hkv)
        return kc, vc, None, None, None, None
    ks_in = np.array([w.k_scalar], np.float32)
    vs_in = np.array([w.v_scalar], np.float32)
    for b in range(w.B):
        k, v, s = w.request_kv(b)
        if w.mode == wl.SCALAR:
            owr.quant_write_ref(k, v, s, kc, vc, ks_in, vs_in, w.mode, w.Hkv)
        else:
            owr.quant_write_ref(k, v, s, kc, vc, ks, vs, w.mode, w.Hkv)
    if w.mode == wl.SCALAR:
        return kc, vc, ks, vs, ks_in, vs_in
    if w.mode == wl.NONE:
        return kc, vc, ks, vs, None, None
    return kc, vc, ks, vs, ks, vs


def oracle_out(w, cache=None, rows_subset=None, sm_scale=None):
    cache = oracle_cache(w) if cache is None else cache
    kc, vc, _, _, ksa, vsa = cache
    return oatt.attention_ref(w.q, kc, vc, ksa, vsa, w.block_table, w.ctx, w.cu, w.sparse, w.mode,
                              w.Hkv, sm_scale=sm_scale, rows_subset=rows_subset, kv_dtype=w.kv_dtype)


def compact_request_cache(w, b):
    """The oracle's compact cache of request b of a large workload: its
    written pages only, logical page n at compact page ``cpage[n]``.
    Returns (kc, vc, ks, vs, ksa, vsa, bt) with ``bt`` the compact block
    table [1, W] and ksa/vsa the scale arguments for the oracle's decode."""
    pages = [int(n) for n in w.written[b]]
    nb = len(pages)
    Hkv = w.Hkv
    bf = w.kv_dtype == "bf16"
    kc = np.zeros(nb * Hkv * 16384, np.uint16 if bf else np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros(nb * Hkv * 128, np.float32)
    vs = np.zeros_like(ks)
    ks_in = np.array([w.k_scalar], np.float32)
    vs_in = np.array([w.v_scalar], np.float32)
    bt = np.full((1, w.W), -1, np.int64)
    for ci, n in enumerate(pages):
        bt[0, n] = ci
        k, v = w.page_kv(b, n)
        slots = ci * 128 + np.arange(k.shape[0], dtype=np.int64)
        if bf:
            owr.write_bf16_ref(k, v, slots, kc, vc, Hkv)
        elif w.mode == wl.SCALAR:
            owr.quant_write_ref(k, v, slots, kc, vc, ks_in, vs_in, w.mode, Hkv)
        else:
            owr.quant_write_ref(k, v, slots, kc, vc, ks, vs, w.mode, Hkv)
    ksa, vsa = (ks_in, vs_in) if w.mode == wl.SCALAR else ((None, None) if w.mode == wl.NONE else (ks, vs))
    return kc, vc, ks, vs, ksa, vsa, bt


def compact_request_oracle(w, b, rows, cc=None):
    """Oracle output for some rows of request b of a large workload, built on
    a compact cache that holds only request b's written pages."""
    kc, vc, ks, vs, ksa, vsa, bt = compact_request_cache(w, b) if cc is None else cc
    start = int(w.row_start[b])
    L = int(w.q_lens[b])
    q = w.q[start:start + L]
    cu = None if w.cu is None else np.array([0, L])
    sp = None if w.sparse is None else w.sparse[start:start + L]
    sel = [r - start for r in rows]
    return oatt.attention_ref(q, kc, vc, ksa, vsa, bt, w.ctx[b:b + 1], cu, sp, w.mode, w.Hkv,
                              rows_subset=sel, kv_dtype=w.kv_dtype)


def assert_request_bytes(w, b, case, cc):
    """The GPU cache's bytes of every written slot of request b's pages (and
    their per-token scale bits) equal the oracle writer's, page by page.
    Slots a page does not hold (the tail of the last page) are not the
    writer's output and are skipped."""
    assert w.kv_dtype == "fp8"
    kc, vc, ks, vs, _, _, bt = cc
    pages = [int(n) for n in w.written[b]]
    phys = torch.as_tensor([int(w.block_table[b, n]) for n in pages], device=case.kc.device)
    gk = case.kc.view(torch.uint8).index_select(0, phys).cpu().numpy()
    gv = case.vc.view(torch.uint8).index_select(0, phys).cpu().numpy()
    Hkv = w.Hkv
    ok = np.reshape(kc, (-1, Hkv, 16384))
    ov = np.reshape(vc, (-1, Hkv, 16384))
    gks = gvs = None
    if w.mode == wl.PER_TOKEN:
        gks = case.ks.index_select(0, phys).cpu().numpy().view(np.uint32)
        gvs = case.vs.index_select(0, phys).cpu().numpy().view(np.uint32)
        oks = np.reshape(ks, (-1, Hkv, 128)).view(np.uint32)
        ovs = np.reshape(vs, (-1, Hkv, 128)).view(np.uint32)
    for i, n in enumerate(pages):
        ci = int(bt[0, n])
        cnt = int(min(128, int(w.ctx[b]) - 128 * n))
        if cnt == 128:
            kidx = vidx = slice(None)
        else:
            o = np.arange(cnt)[:, None]
            d = np.arange(128)[None, :]
            kidx = olay.k_offset(o, d).reshape(-1)
            vidx = olay.v_offset(o, d).reshape(-1)
        for h in range(Hkv):
            assert np.array_equal(gk[i, h][kidx], ok[ci, h][kidx]), f"request {b} page {n} head {h}: K bytes"
            assert np.array_equal(gv[i, h][vidx], ov[ci, h][vidx]), f"request {b} page {n} head {h}: V bytes"
            if gks is not None:
                assert np.array_equal(gks[i, h, :cnt], oks[ci, h, :cnt]), f"request {b} page {n}: K scales"
                assert np.array_equal(gvs[i, h, :cnt], ovs[ci, h, :cnt]), f"request {b} page {n}: V scales"


def compare(gpu_bf16, ref64, atol=1e-2, cos_min=0.9999, what=""):
    """Element-wise parity of a bf16 output with the fp64 oracle: |err| <=
    atol (1e-2) wherever |ref| < 4, and 2^-7 |ref| where |ref| >= 4 -- there
    half a bf16 ulp alone is at least 2^-6 = 0.0156 > 1e-2, so no bf16 value
    can meet the absolute bound; 2^-7 |ref| is one ulp at the bottom of the
    binade.  Plus cosine >= cos_min over the whole tensor."""
    g = gpu_bf16.float().cpu().numpy().astype(np.float64) if torch.is_tensor(gpu_bf16) else gpu_bf16
    r = np.asarray(ref64, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    maxerr = float(err.max()) if err.size else 0.0
    mag = np.abs(r)
    relaxed = mag >= 4.0
    tol = np.where(relaxed, 2.0 ** -7 * mag, atol)
    worst = float((err / tol).max()) if err.size else 0.0
    num = float(np.sum(g * r))
    den = math.sqrt(float(np.sum(g * g)) * float(np.sum(r * r)))
    cos = num / den if den > 0 else (1.0 if float(np.abs(g).max(initial=0)) == 0 else 0.0)
    maxref = float(mag.max()) if mag.size else 0.0
    abs_err = float(err[~relaxed].max()) if np.any(~relaxed) else 0.0
    assert worst <= 1.0, (f"{what}: max|err| {maxerr:.3e} (where |ref| < 4: {abs_err:.3e}) exceeds the "
                          f"bound ({atol} for |ref| < 4, 2^-7|ref| above; max|ref| {maxref:.3e}, "
                          f"{int(relaxed.sum())} of {r.size} elements at |ref| >= 4, worst err/tol "
                          f"{worst:.3f})")
    assert cos >= cos_min, f"{what}: cosine {cos:.7f} < {cos_min}"
    return maxerr, cos
