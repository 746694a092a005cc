"""Host-only checks of the C ABI (no GPU needed): the library loads and
exports every entry point include/fp8pa.h declares; configuration checks,
capacity buckets and refusals happen on the host before any launch."""

import ctypes
import os
import re

import pytest
import torch

import fp8_paged_kv_pa_amd as pa
from fp8_paged_kv_pa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8pa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names


def test_library_exports_every_declared_symbol():
    lib = pa.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_struct_sizes_match_header_layout():
    # pa_tensor: ptr + 2 x int32 + 12 x int64
    assert ctypes.sizeof(_lib.PaTensor) == 8 + 8 + 6 * 8 * 2
    assert ctypes.sizeof(_lib.PaConfig) == 6 * 4 + 4 * 8 + 5 * 4 + 4  # tail padded to 8
    assert ctypes.sizeof(_lib.PaDecodeOpts) == 4 + 4 + 4 + 4 + 8 + 8 + 4 + 4 + 4 + 4
    assert ctypes.sizeof(_lib.PaPlanInfo) == 4 * 4 + 6 * 8 + 3 * 4 + 4  # tail padded to 8


def cfg(**kw):
    base = dict(num_kv_heads=1, rows=4, batch=4, max_pages=72)
    base.update(kw)
    return pa.make_config(**base)


@pytest.mark.parametrize("field,value,status", [
    ("group_size", 8, -5), ("head_dim", 64, -5), ("page_size", 16, -5),
    ("num_kv_heads", 0, -5), ("kv_dtype", 4, -2), ("scale_mode", 7, -1),
])
def test_geometry_refused_up_front(field, value, status):
    c = cfg()
    setattr(c, field, value)
    assert pa.pa_query_support(c) == status
    assert pa.pa_last_error()


def test_bf16_cache_only_without_scales():
    """The unquantized bf16 cache is served with scale_mode NONE only."""
    assert pa.pa_query_support(cfg(kv_dtype=3, scale_mode=pa.SCALE_NONE)) == 0
    assert pa.pa_query_support(cfg(kv_dtype=3, scale_mode=pa.SCALE_PER_TOKEN)) == -5
    assert "unquantized" in pa.pa_last_error()
    assert pa.pa_query_support(cfg(kv_dtype=3, scale_mode=pa.SCALE_SCALAR)) == -5
    # same plan and scratch as the FP8 cache of the same shape
    a = pa.pa_plan_describe(cfg(kv_dtype=3, scale_mode=pa.SCALE_NONE, rows=124, batch=31, max_pages=256))
    b = pa.pa_plan_describe(cfg(rows=124, batch=31, max_pages=256))
    assert a == b


def test_non_divisible_rows_without_cu_is_refused():
    # 121 rows over 31 requests: only a ragged (cu_seqlens_q) call may take it
    assert pa.pa_query_support(cfg(rows=121, batch=31)) == -3
    assert "cu_seqlens_q" in pa.pa_last_error()
    assert pa.pa_query_support(cfg(rows=121, batch=31, ragged=True)) == 0
    # [4,4,6,2]: divisible by 4, but with cu it is planned as ragged (max q_len unknown -> rows)
    p = pa.pa_plan_describe(cfg(rows=16, batch=4, ragged=True))
    assert p["rows_per_group"] == 2 and p["groups"] == 8
    p = pa.pa_plan_describe(cfg(rows=16, batch=4, ragged=True, max_q_len=6))
    assert p["rows_per_group"] == 2 and p["groups"] == 3
    p = pa.pa_plan_describe(cfg(rows=16, batch=16))
    assert p["rows_per_group"] == 1 and p["groups"] == 1


def test_capacity_refusals():
    assert pa.pa_query_support(cfg(rows=65537, batch=1)) == -6
    assert pa.pa_query_support(cfg(rows=65536, batch=65536, max_pages=1)) == 0
    assert pa.pa_query_support(cfg(topk=5000, rows=4)) == -6
    assert pa.pa_query_support(cfg(max_pages=(1 << 20) + 1)) == -6


def test_grid_beyond_one_launch_is_refused():
    """A ragged call with no max_q_len plans every request as rows long; with
    many requests that needs more than 2^31 - 1 workgroups: refused with a
    pointer to max_q_len, never truncated."""
    big = cfg(rows=65536, batch=65536, ragged=True, max_pages=1024, num_kv_heads=64)
    assert pa.pa_query_support(big) == -6
    assert "max_q_len" in pa.pa_last_error()
    assert pa.pa_query_support(cfg(rows=65536, batch=65536, ragged=True, max_pages=1024, num_kv_heads=64,
                                   max_q_len=1)) == 0


def test_plans_and_scratch_depend_only_on_buckets():
    """Every row count inside one power-of-two bucket maps to the same
    partition count and scratch size; the set of scratch sizes is bounded by
    the number of buckets (not by the number of distinct row counts)."""
    sizes = set()
    for rows in range(1, 4097):
        p = pa.pa_plan_describe(cfg(rows=rows, batch=rows, max_pages=1024))
        bucket = 1 << (rows - 1).bit_length()
        assert p["rows_bucket"] == bucket
        sizes.add(p["scratch_bytes"])
    assert len(sizes) <= 13
    a = pa.pa_plan_describe(cfg(rows=33, batch=33, max_pages=1024))
    b = pa.pa_plan_describe(cfg(rows=64, batch=64, max_pages=1024))
    assert a["scratch_bytes"] == b["scratch_bytes"] and a["parts"] == b["parts"]


def test_plan_shapes_for_the_workloads():
    c2 = pa.pa_plan_describe(cfg(rows=4, batch=4, max_pages=72))
    assert c2["merge"] == 1 and c2["pages_per_part"] >= 1 and c2["units"] == 4
    assert c2["balanced"] == 0  # two pages per partition: the fixed split
    c3f = pa.pa_plan_describe(cfg(rows=32, batch=32, max_pages=1024, partition_mode=pa.PARTITION_FIXED))
    assert c3f["parts"] * c3f["pages_per_part"] >= 1024 and c3f["grid_x"] == 32 * c3f["parts"]
    assert c3f["balanced"] == 0
    # length-balanced: 256 slots shared by the 32 requests, sizes chosen on the device
    c3 = pa.pa_plan_describe(cfg(rows=32, batch=32, max_pages=1024))
    assert c3["balanced"] == 1 and c3["parts"] == 256 and c3["pages_per_part"] == 0
    assert c3["grid_x"] == 256 and c3["merge"] == 1 and c3["merge_in_kernel"] == 0
    c4 = pa.pa_plan_describe(cfg(rows=124, batch=31, max_pages=256))
    assert c4["balanced"] == 1 and c4["groups"] == 2 and c4["parts"] == 128 and c4["grid_x"] == 256
    c4r = pa.pa_plan_describe(cfg(rows=121, batch=31, max_pages=256, ragged=True))
    assert c4r["balanced"] == 0  # ragged without max_q_len: fixed
    c4m = pa.pa_plan_describe(cfg(rows=121, batch=31, max_pages=256, ragged=True, max_q_len=4))
    assert c4m["balanced"] == 1
    big = pa.pa_plan_describe(cfg(rows=65, batch=65, max_pages=1024))
    assert big["balanced"] == 0  # more than 64 requests
    assert pa.pa_query_support(cfg(rows=65, batch=65, max_pages=1024, partition_mode=pa.PARTITION_BALANCED)) == -5
    assert pa.pa_query_support(cfg(topk=8, partition_mode=pa.PARTITION_BALANCED)) == -5
    assert pa.pa_query_support(cfg(partition_mode=3)) == -1
    c5 = pa.pa_plan_describe(cfg(rows=16, batch=16, max_pages=1024, topk=32))
    assert c5["units"] == 16 and c5["parts"] * c5["pages_per_part"] >= 32
    one = pa.pa_plan_describe(cfg(rows=4, batch=4, max_pages=72, force_parts=1))
    assert one["merge"] == 0 and one["scratch_bytes"] == 0
    dflt = pa.pa_plan_describe(cfg(rows=4, batch=4, max_pages=72))
    fused = pa.pa_plan_describe(cfg(rows=4, batch=4, max_pages=72, merge_mode=pa.MERGE_IN_KERNEL))
    sep = pa.pa_plan_describe(cfg(rows=4, batch=4, max_pages=72, merge_mode=pa.MERGE_SEPARATE))
    assert fused["merge_in_kernel"] == 1 and sep["merge_in_kernel"] == 0 and dflt["merge_in_kernel"] == 0
    assert fused["scratch_bytes"] == sep["scratch_bytes"]
    assert pa.pa_query_support(cfg(merge_mode=3)) == -1


def _host_tensor(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def _decode_args(**over):
    t = dict(
        q=_host_tensor((4, 16, 128), torch.bfloat16),
        k=_host_tensor((8, 1, 16384), torch.uint8),
        v=_host_tensor((8, 1, 16384), torch.uint8),
        ks=_host_tensor((8, 1, 128), torch.float32),
        vs=_host_tensor((8, 1, 128), torch.float32),
        bt=_host_tensor((4, 2), torch.int32),
        ctx=_host_tensor((4,), torch.int32),
        cu=None, sp=None,
        out=_host_tensor((4, 16, 128), torch.bfloat16),
        mode=2,
    )
    t.update(over)
    return t


def _call_decode(t):
    lib = pa.load()
    d = [_lib.desc(t[k]) for k in ("q", "k", "v", "ks", "vs", "bt", "ctx", "cu", "sp")]
    do = _lib.desc(t["out"])
    return lib.pa_decode(*[_lib.ref(x) for x in d], t["mode"], _lib.ref(do), None)


@pytest.mark.parametrize("over,status", [
    (dict(q=_host_tensor((4, 16, 128), torch.float32)), -2),
    (dict(q=_host_tensor((4, 16, 64), torch.bfloat16)), -5),
    (dict(q=_host_tensor((4, 32, 128), torch.bfloat16)), -5),
    (dict(k=_host_tensor((8, 1, 8192), torch.uint8)), -3),
    (dict(v=_host_tensor((8, 1, 16384), torch.float32)), -2),
    (dict(ks=_host_tensor((8, 1, 64), torch.float32)), -3),
    (dict(ks=_host_tensor((8, 1, 128), torch.float32), mode=1), -3),
    (dict(bt=_host_tensor((4, 2), torch.int64)), -2),
    (dict(ctx=_host_tensor((3,), torch.int32)), -3),
    (dict(cu=_host_tensor((4,), torch.int32)), -3),
    (dict(sp=_host_tensor((3, 4), torch.int32)), -3),
    (dict(out=_host_tensor((4, 16, 128), torch.float32)), -3),
    (dict(q=_host_tensor((6, 16, 128), torch.bfloat16), out=_host_tensor((6, 16, 128), torch.bfloat16)), -3),
    (dict(q=_host_tensor((4, 16, 130), torch.bfloat16)[:, :, :128]), -4),
    (dict(mode=5), -1),
    # bf16 caches: 16384 elements per block, no scales, both caches alike
    (dict(k=_host_tensor((8, 1, 16384), torch.bfloat16), v=_host_tensor((8, 1, 16384), torch.bfloat16)), -5),
    (dict(k=_host_tensor((8, 1, 16384), torch.bfloat16)), -2),
    (dict(k=_host_tensor((8, 1, 8192), torch.bfloat16), v=_host_tensor((8, 1, 8192), torch.bfloat16),
          mode=0), -3),
])
def test_decode_refuses_bad_descriptors_before_launch(over, status):
    assert _call_decode(_decode_args(**over)) == status
    assert pa.pa_last_error()


def test_decode_accepts_bf16_cache_descriptors_on_the_host():
    """A well-formed bf16-cache call passes every host check; with zero
    rows nothing is launched, so this runs without a GPU."""
    t = _decode_args(q=_host_tensor((0, 16, 128), torch.bfloat16),
                     out=_host_tensor((0, 16, 128), torch.bfloat16),
                     k=_host_tensor((8, 1, 16384), torch.bfloat16),
                     v=_host_tensor((8, 1, 16384), torch.bfloat16), ks=None, vs=None, mode=0)
    assert _call_decode(t) == 0, pa.pa_last_error()


def test_write_refuses_bad_descriptors_before_launch():
    lib = pa.load()
    k = _host_tensor((3, 1, 128), torch.float32)
    slots = _host_tensor((3,), torch.int32)  # wrong dtype: must be int64
    kc = _host_tensor((2, 1, 16384), torch.uint8)
    ks = _host_tensor((2, 1, 128), torch.float32)
    d = [_lib.desc(x) for x in (k, k, slots, kc, kc, ks, ks)]
    assert lib.kv_quant_write(*[_lib.ref(x) for x in d], 2, None) == -3
    k2 = _host_tensor((3, 2, 128), torch.float32)
    d = [_lib.desc(x) for x in (k2, k2, _host_tensor((3,), torch.int64), kc, kc, ks, ks)]
    assert lib.kv_quant_write(*[_lib.ref(x) for x in d], 2, None) == -3
    assert "KV heads" in pa.pa_last_error()


def test_write_to_bf16_cache_refuses_scales():
    lib = pa.load()
    k = _host_tensor((3, 1, 128), torch.float32)
    slots = _host_tensor((3,), torch.int64)
    kc = _host_tensor((2, 1, 16384), torch.bfloat16)
    ks = _host_tensor((2, 1, 128), torch.float32)
    d = [_lib.desc(x) for x in (k, k, slots, kc, kc, ks, ks)]
    assert lib.kv_quant_write(*[_lib.ref(x) for x in d], 2, None) == -5
    u8 = _host_tensor((2, 1, 16384), torch.uint8)
    d = [_lib.desc(x) for x in (k, k, slots, kc, u8, ks, ks)]
    assert lib.kv_quant_write(*[_lib.ref(x) for x in d], 0, None) == -2


def _index_args(**over):
    t = dict(
        q=_host_tensor((4, 128), torch.bfloat16),
        cache=_host_tensor((8, 128, 128), torch.uint8),
        bt=_host_tensor((4, 3), torch.int32),
        ctx=_host_tensor((4,), torch.int32),
        cu=None,
        idx=_host_tensor((4, 32), torch.int32),
        scores=_host_tensor((4, 3), torch.float32),
        max_q_len=0,
    )
    t.update(over)
    return t


def _call_index(t):
    lib = pa.load()
    d = [_lib.desc(t[k]) for k in ("q", "cache", "bt", "ctx", "cu")]
    di, ds = _lib.desc(t["idx"]), _lib.desc(t["scores"])
    return lib.pa_index_topk(*[_lib.ref(x) for x in d], t["max_q_len"], 0.0, _lib.ref(di), _lib.ref(ds), None)


@pytest.mark.parametrize("over,status", [
    (dict(q=_host_tensor((4, 128), torch.float32)), -2),
    (dict(q=_host_tensor((4, 64), torch.bfloat16)), -3),
    (dict(cache=_host_tensor((8, 128, 64), torch.uint8)), -3),
    (dict(cache=_host_tensor((8, 128, 128), torch.bfloat16)), -2),
    (dict(bt=_host_tensor((4, 3), torch.int64)), -2),
    (dict(ctx=_host_tensor((3,), torch.int32)), -3),
    (dict(q=_host_tensor((6, 128), torch.bfloat16), idx=_host_tensor((6, 32), torch.int32),
          scores=_host_tensor((6, 3), torch.float32)), -3),  # 6 rows over 4 requests, no cu
    (dict(idx=_host_tensor((4, 0), torch.int32)), -3),
    (dict(idx=_host_tensor((4, 5000), torch.int32)), -6),
    (dict(scores=_host_tensor((4, 4), torch.float32)), -3),
    (dict(max_q_len=-1), -1),
])
def test_index_topk_refuses_bad_descriptors_before_launch(over, status):
    assert _call_index(_index_args(**over)) == status
    assert pa.pa_last_error()


def test_index_topk_accepts_a_well_formed_empty_call():
    t = _index_args(q=_host_tensor((0, 128), torch.bfloat16), idx=_host_tensor((0, 32), torch.int32),
                    scores=_host_tensor((0, 3), torch.float32))
    assert _call_index(t) == 0, pa.pa_last_error()


def _call_check(t, report):
    lib = pa.load()
    d = [_lib.desc(t[k]) for k in ("q", "k", "v", "ks", "vs", "bt", "ctx", "cu", "sp")]
    do = _lib.desc(t["out"])
    return lib.pa_check_decode_inputs(*[_lib.ref(x) for x in d], t["mode"], _lib.ref(do), report, None)


@pytest.mark.parametrize("over,status", [
    (dict(q=_host_tensor((4, 16, 128), torch.float32)), -2),
    (dict(ctx=_host_tensor((3,), torch.int32)), -3),
    (dict(sp=_host_tensor((3, 4), torch.int32)), -3),
    (dict(q=_host_tensor((6, 16, 128), torch.bfloat16), out=_host_tensor((6, 16, 128), torch.bfloat16)), -3),
    (dict(mode=5), -1),
])
def test_input_check_runs_the_decode_host_validation_first(over, status):
    # the same host checks as pa_decode, before anything is launched (the
    # report pointer is never touched on these paths)
    assert _call_check(_decode_args(**over), ctypes.c_void_p(0x10000)) == status
    assert pa.pa_last_error()


def test_input_check_needs_a_report_buffer():
    assert _call_check(_decode_args(), None) == -1
    assert "report" in pa.pa_last_error()


def _call_noalloc(t, **opts):
    lib = pa.load()
    d = [_lib.desc(t[k]) for k in ("q", "k", "v", "ks", "vs", "bt", "ctx", "cu", "sp")]
    do = _lib.desc(t["out"])
    o = _lib.PaDecodeOpts()
    for k, v in opts.items():
        setattr(o, k, v)
    return lib.pa_decode_noalloc(*[_lib.ref(x) for x in d], t["mode"], _lib.ref(do), ctypes.byref(o), None)


@pytest.mark.parametrize("over,status", [
    (dict(q=_host_tensor((4, 16, 128), torch.float32)), -2),
    (dict(k=_host_tensor((8, 1, 8192), torch.uint8)), -3),
    (dict(ctx=_host_tensor((3,), torch.int32)), -3),
    (dict(mode=5), -1),
])
def test_noalloc_runs_the_decode_host_validation(over, status):
    assert _call_noalloc(_decode_args(**over)) == status
    assert pa.pa_last_error()


def test_noalloc_refusals_before_any_device_call():
    # the in-kernel merge needs zeroed counters the fixed array does not keep
    assert _call_noalloc(_decode_args(), force_parts=4, merge_mode=pa.MERGE_IN_KERNEL) == -5
    assert "in-kernel merge" in pa.pa_last_error()
    # 16384 one-row requests at 8 partitions: a scratch bucket above the 32 MiB array
    T = 16384
    t = _decode_args(q=_host_tensor((T, 16, 128), torch.bfloat16), out=_host_tensor((T, 16, 128), torch.bfloat16),
                     bt=_host_tensor((T, 2), torch.int32), ctx=_host_tensor((T,), torch.int32))
    assert _call_noalloc(t, force_parts=2) == -6
    assert "pa_decode_noalloc" in pa.pa_last_error()
    # a well-formed empty call passes every check and launches nothing
    e = _decode_args(q=_host_tensor((0, 16, 128), torch.bfloat16), out=_host_tensor((0, 16, 128), torch.bfloat16))
    assert _call_noalloc(e) == 0, pa.pa_last_error()


def _norm_rope_call(T=3, with_q=True, **over):
    lib = pa.load()
    t = dict(
        q=_host_tensor((T, 16, 128), torch.float32) if with_q else None,
        q_out=_host_tensor((T, 16, 128), torch.bfloat16) if with_q else None,
        k=_host_tensor((T, 1, 128), torch.float32), v=_host_tensor((T, 1, 128), torch.float32),
        slots=_host_tensor((T,), torch.int64),
        kc=_host_tensor((2, 1, 16384), torch.uint8), vc=_host_tensor((2, 1, 16384), torch.uint8),
        ks=_host_tensor((2, 1, 128), torch.float32), vs=_host_tensor((2, 1, 128), torch.float32),
        pos=_host_tensor((T,), torch.int64), cos=_host_tensor((64, 32), torch.float32),
        sin=_host_tensor((64, 32), torch.float32), kw=_host_tensor((128,), torch.float32), qw=None,
        rot=64, neox=1, eps=1e-6, off=1.0, nr=True)
    t.update(over)
    keep = [_lib.desc(t[k]) for k in ("pos", "cos", "sin", "kw", "qw")]
    nr = _lib.PaNormRope()
    nr.positions, nr.cos, nr.sin, nr.k_norm_weight, nr.q_norm_weight = [
        None if x is None else ctypes.pointer(x) for x in keep]
    nr.rotary_dim, nr.neox, nr.eps, nr.weight_offset = t["rot"], t["neox"], t["eps"], t["off"]
    d = [_lib.desc(t[k]) for k in ("q", "q_out", "k", "v", "slots", "kc", "vc", "ks", "vs")]
    return lib.kv_norm_rope_write(*[_lib.ref(x) for x in d], 2, ctypes.byref(nr) if t["nr"] else None, None)


@pytest.mark.parametrize("over,status", [
    (dict(rot=6), -5),
    (dict(rot=132), -5),
    (dict(cos=_host_tensor((64, 16), torch.float32)), -3),
    (dict(sin=_host_tensor((32, 32), torch.float32)), -3),
    (dict(pos=_host_tensor((3,), torch.int32)), -3),
    (dict(pos=_host_tensor((4,), torch.int64)), -3),
    (dict(kw=_host_tensor((64,), torch.float32)), -3),
    (dict(qw=_host_tensor((128,), torch.bfloat16)), -3),
    (dict(eps=-1.0), -1),
    (dict(eps=float("inf")), -1),
    (dict(off=float("nan")), -1),
    (dict(q_out=None), -1),
    (dict(q=_host_tensor((3, 8, 128), torch.float32), q_out=_host_tensor((3, 8, 128), torch.bfloat16)), -3),
    (dict(q_out=_host_tensor((3, 16, 128), torch.float32)), -2),
    (dict(nr=False), -1),
])
def test_fused_writer_refuses_bad_arguments_before_launch(over, status):
    assert _norm_rope_call(**over) == status
    assert pa.pa_last_error()


def test_fused_writer_accepts_well_formed_empty_calls():
    assert _norm_rope_call(T=0) == 0, pa.pa_last_error()
    # no rotation: the tables may be absent
    assert _norm_rope_call(T=0, with_q=False, rot=0, cos=None, sin=None, kw=None) == 0, pa.pa_last_error()


def _call_decode_write(t, T=4, kdt=torch.float32, slot_dtype=torch.int64, **opts):
    lib = pa.load()
    kn = _host_tensor((T, 1, 128), kdt)
    sl = _host_tensor((T,), slot_dtype)
    d = [_lib.desc(x) for x in (t["q"], kn, kn, sl, t["k"], t["v"], t["ks"], t["vs"], t["bt"], t["ctx"], t["cu"],
                                None)]
    do = _lib.desc(t["out"])
    o = _lib.PaDecodeOpts()
    for k, v in opts.items():
        setattr(o, k, v)
    return lib.pa_decode_write(*[_lib.ref(x) for x in d], t["mode"], _lib.ref(do), ctypes.byref(o), None)


@pytest.mark.parametrize("over,kw,status,text", [
    (dict(), dict(T=3), -3, "query rows"),                                   # one new token per query row
    (dict(), dict(kdt=torch.int32), -2, "k_new"),                            # writer inputs f32 / bf16
    (dict(), dict(slot_dtype=torch.int32), -3, "slot_mapping"),
    (dict(bt=_host_tensor((4, 2), torch.int64)), dict(), -2, "block_table"),  # the decode's own checks
    (dict(mode=5), dict(), -1, "scale_mode"),
])
def test_decode_write_refuses_bad_arguments_before_launch(over, kw, status, text):
    assert _call_decode_write(_decode_args(**over), **kw) == status
    assert text in pa.pa_last_error()


def test_decode_write_accepts_a_well_formed_empty_call():
    e = _decode_args(q=_host_tensor((0, 16, 128), torch.bfloat16), out=_host_tensor((0, 16, 128), torch.bfloat16))
    assert _call_decode_write(e, T=0) == 0, pa.pa_last_error()
