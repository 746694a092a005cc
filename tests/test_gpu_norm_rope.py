"""GPU parity of kv_norm_rope_write (the cache writer fused with the key's
RMS norm and rotary embedding, and the query's) against the oracle's fp32
reading: every cache byte, every scale bit and every bf16 bit of the
transformed query equal the oracle's, over seeded random calls; and a
decode over the cache it wrote matches the oracle's attention."""

import numpy as np
import pytest
import torch

import fp8_paged_kv_pa_amd as pa
import workloads as wl
from oracle import attention as oatt
from oracle import norm_rope as onr

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 200))
    Hkv = int(rng.integers(1, 4))
    nb = int(rng.integers(2, 5))
    kv_dtype = "bf16" if rng.random() < 0.2 else "fp8"
    mode = wl.NONE if kv_dtype == "bf16" else [wl.PER_TOKEN, wl.SCALAR, wl.NONE][int(rng.integers(0, 3))]
    rot = int(rng.choice([0, 4, 32, 64, 96, 128]))
    neox = bool(rng.random() < 0.5)
    bf16_in = bool(rng.random() < 0.4)
    mag = 10.0 ** rng.uniform(-3, 3, size=(T, Hkv, 1))
    k = (rng.standard_normal((T, Hkv, 128)) * mag).astype(np.float32)
    v = (rng.standard_normal((T, Hkv, 128)) * mag).astype(np.float32)
    q = (rng.standard_normal((T, 16 * Hkv, 128)) * 3).astype(np.float32)
    k[rng.random(T) < 0.05] = 0.0
    if bf16_in:
        k, v, q = wl.bf16_round(k), wl.bf16_round(v), wl.bf16_round(q)
    slots = rng.permutation(nb * 128)[:T].astype(np.int64)
    if T > nb * 128:
        slots = np.concatenate([slots, np.full(T - nb * 128, -1, np.int64)])
    slots[rng.random(T) < 0.1] = -1
    max_pos = int(rng.integers(1, 600))
    pos = rng.integers(-3, max_pos + 5, size=T).astype(np.int64)    # a few outside the table
    c, s = wl.rope_tables(max_pos, max(rot, 4), base=float(rng.choice([10000.0, 1e6])))
    kw = (rng.standard_normal(128) * 0.2).astype(np.float32) if rng.random() < 0.7 else None
    qw = (rng.standard_normal(128) * 0.2).astype(np.float32) if rng.random() < 0.7 else None
    with_q = bool(rng.random() < 0.7)
    eps = float(np.float32(rng.choice([1e-6, 1e-5, 0.1])))
    off = float(rng.choice([0.0, 1.0]))
    return dict(T=T, Hkv=Hkv, nb=nb, kv_dtype=kv_dtype, mode=mode, rot=rot, neox=neox, bf16_in=bf16_in,
                k=k, v=v, q=q if with_q else None, slots=slots, pos=pos, c=c, s=s, kw=kw, qw=qw, eps=eps,
                off=off, rng=rng)


def _run(d):
    dev = torch.device("cuda:0")
    T, Hkv, nb, rng = d["T"], d["Hkv"], d["nb"], d["rng"]
    bf = d["kv_dtype"] == "bf16"
    if bf:
        kc0 = rng.integers(0, 1 << 16, size=nb * Hkv * 16384, dtype=np.uint16)
        vc0 = rng.integers(0, 1 << 16, size=nb * Hkv * 16384, dtype=np.uint16)
    else:
        kc0 = rng.integers(0, 256, size=nb * Hkv * 16384, dtype=np.uint8)
        vc0 = rng.integers(0, 256, size=nb * Hkv * 16384, dtype=np.uint8)
    s0 = np.full(nb * Hkv * 128, -3.0, np.float32)
    tdt = torch.int16 if bf else torch.uint8
    kc_g = torch.from_numpy(kc0.view(np.int16) if bf else kc0.copy()).to(dev).view(nb, Hkv, 16384)
    vc_g = torch.from_numpy(vc0.view(np.int16) if bf else vc0.copy()).to(dev).view(nb, Hkv, 16384)
    if bf:
        kc_g, vc_g = kc_g.view(torch.bfloat16), vc_g.view(torch.bfloat16)
    mode = d["mode"]
    if mode == wl.SCALAR:
        sk, sv = np.float32(rng.uniform(1e-3, 1)), np.float32(rng.uniform(1e-3, 1))
        ks_g, vs_g = torch.tensor([sk], device=dev), torch.tensor([sv], device=dev)
    elif mode == wl.PER_TOKEN:
        ks_g = torch.from_numpy(s0.copy()).to(dev).view(nb, Hkv, 128)
        vs_g = torch.from_numpy(s0.copy()).to(dev).view(nb, Hkv, 128)
    else:
        ks_g = vs_g = None
    tin = torch.bfloat16 if d["bf16_in"] else torch.float32
    g = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    q_out = None if d["q"] is None else torch.empty(T, 16 * Hkv, 128, dtype=torch.bfloat16, device=dev)
    pa.kv_norm_rope_write(g(d["k"]).to(tin), g(d["v"]).to(tin), g(d["slots"]), kc_g, vc_g, ks_g, vs_g, mode,
                          g(d["pos"]), g(d["c"]), g(d["s"]), d["rot"], d["neox"], g(d["kw"]), g(d["qw"]),
                          d["eps"], d["off"], None if d["q"] is None else g(d["q"]).to(tin), q_out)
    torch.cuda.synchronize()
    kc, vc, ks, vs = kc0.copy(), vc0.copy(), s0.copy(), s0.copy()
    if mode == wl.SCALAR:
        ka, va = np.array([sk]), np.array([sv])
    elif mode == wl.PER_TOKEN:
        ka, va = ks, vs
    else:
        ka = va = None
    qbits = onr.norm_rope_write_ref(d["k"], d["v"], d["slots"], d["pos"], d["c"], d["s"], d["rot"], d["neox"],
                                    d["kw"], d["eps"], d["off"], kc, vc, ka, va, mode, Hkv, q=d["q"],
                                    q_weight=d["qw"], kv_dtype=d["kv_dtype"])
    gk = kc_g.view(torch.int16 if bf else torch.uint8).cpu().numpy().reshape(-1)
    gv = vc_g.view(torch.int16 if bf else torch.uint8).cpu().numpy().reshape(-1)
    if bf:
        gk, gv = gk.view(np.uint16), gv.view(np.uint16)
    assert np.array_equal(gk, kc), "K cache"
    assert np.array_equal(gv, vc), "V cache"
    if mode == wl.PER_TOKEN:
        assert np.array_equal(ks_g.cpu().numpy().reshape(-1).view(np.uint32), ks.view(np.uint32)), "K scales"
        assert np.array_equal(vs_g.cpu().numpy().reshape(-1).view(np.uint32), vs.view(np.uint32)), "V scales"
    if q_out is not None:
        assert np.array_equal(q_out.view(torch.int16).cpu().numpy().view(np.uint16), qbits), "q"
    return kc_g, vc_g, ks_g, vs_g


@pytest.mark.parametrize("seed", list(range(1101, 1141)))
def test_fused_write_bit_exact(seed):
    d = _draw(seed)
    print("norm_rope", seed, {k: d[k] for k in ("T", "Hkv", "kv_dtype", "mode", "rot", "neox", "bf16_in",
                                                 "eps", "off")}, "kw", d["kw"] is not None, "q",
          d["q"] is not None, flush=True)
    _run(d)


@pytest.mark.parametrize("rot,neox", [(128, True), (128, False), (64, True)])
def test_edge_rows(rot, neox):
    """Tiny rows (eps dominates), zero rows, huge rows, a row whose norm is
    set by one element; positions at both ends of the table."""
    d = _draw(1199)
    T, Hkv = 8, 1
    k = np.ones((T, Hkv, 128), np.float32)
    k[0] *= np.float32(1e-20)
    k[1] = 0.0
    k[2] *= np.float32(1e18)
    k[3] = 0.0
    k[3, 0, 7] = -3.0
    k[4] = np.linspace(-1, 1, 128, dtype=np.float32)
    k[5:] = np.random.default_rng(1200).standard_normal((3, Hkv, 128)).astype(np.float32)
    c, s = wl.rope_tables(64, rot)
    d.update(T=T, Hkv=Hkv, nb=1, kv_dtype="fp8", mode=wl.PER_TOKEN, rot=rot, neox=neox, bf16_in=False,
             k=k, v=k.copy(), q=np.repeat(k, 16, axis=1), slots=np.arange(T, dtype=np.int64) * 3,
             pos=np.array([0, 63, 1, 62, 5, -1, 64, 10**12]), c=c, s=s,
             kw=np.full(128, 0.5, np.float32), qw=None, eps=1e-6, off=1.0)
    _run(d)


def test_decode_over_the_fused_cache():
    """Write a small context through the fused writer, then decode with the
    transformed queries: matches the oracle's attention over the oracle's
    cache."""
    from harness import compare
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1210)
    ctx = [300, 129]
    B, Hkv, rot = 2, 2, 64
    pages = [(c + 127) // 128 for c in ctx]
    nb = sum(pages) + 1
    bt = np.full((B, max(pages)), -1, np.int32)
    perm = rng.permutation(nb)
    at = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[at:at + pages[b]]
        at += pages[b]
    ks_, vs_, sl, ps = [], [], [], []
    for b in range(B):
        for t in range(ctx[b]):
            sl.append(int(bt[b, t // 128]) * 128 + t % 128)
            ps.append(t)
    T = len(sl)
    k = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    slots, pos = np.array(sl, np.int64), np.array(ps, np.int64)
    c, s = wl.rope_tables(512, rot)
    kw = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    kc_g = torch.zeros(nb, Hkv, 16384, dtype=torch.uint8, device=dev)
    vc_g = torch.zeros_like(kc_g)
    ks_g = torch.zeros(nb, Hkv, 128, dtype=torch.float32, device=dev)
    vs_g = torch.zeros_like(ks_g)
    g = lambda a: torch.from_numpy(a).to(dev)
    pa.kv_norm_rope_write(g(k), g(v), g(slots), kc_g, vc_g, ks_g, vs_g, wl.PER_TOKEN, g(pos), g(c), g(s), rot,
                          True, g(kw), None, 1e-6, 0.0)
    # the step's queries at each request's last position, transformed with the same rotation
    qraw = rng.standard_normal((B, 1, 16 * Hkv, 128)).astype(np.float32)
    qpos = np.array([ctx[0] - 1, ctx[1] - 1])
    qt = np.stack([onr.norm_rope_f32(qraw[b], qpos[b:b + 1], c, s, rot, True) for b in range(B)])[:, 0]
    q_bf = wl.bf16_round(qt)
    out = torch.empty(B, 16 * Hkv, 128, dtype=torch.bfloat16, device=dev)
    pa.pa_decode(g(q_bf).to(torch.bfloat16), kc_g, vc_g, ks_g, vs_g, g(bt), g(np.array(ctx, np.int32)), None,
                 None, wl.PER_TOKEN, out)
    torch.cuda.synchronize()
    kc = np.zeros(nb * Hkv * 16384, np.uint8)
    vc = kc.copy()
    ks = np.zeros(nb * Hkv * 128, np.float32)
    vs = ks.copy()
    onr.norm_rope_write_ref(k, v, slots, pos, c, s, rot, True, kw, 1e-6, 0.0, kc, vc, ks, vs, wl.PER_TOKEN, Hkv)
    assert np.array_equal(kc_g.cpu().numpy().reshape(-1), kc)
    ref = oatt.attention_ref(q_bf, kc, vc, ks, vs, bt, np.array(ctx), None, None, wl.PER_TOKEN, Hkv)
    compare(out, ref, what="decode over the fused cache")
