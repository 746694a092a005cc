"""fp8_paged_kv_pa_amd -- paged decode attention over a page-shuffled FP8
(e4m3fn) KV cache with per-token K/V scales, for MI355X (gfx950).

A thin Python face of the C ABI in ``include/fp8pa.h`` (same names).  The
functions here only marshal torch tensors into descriptors; all work runs in
the HIP kernels of ``libfp8pa.so``.  PyTorch supplies device memory and the
stream.
"""

import ctypes

import torch

from ._lib import (  # noqa: F401
    EXPORTS, MERGE_IN_KERNEL, MERGE_PLAN, MERGE_SEPARATE, PARTITION_BALANCED, PARTITION_FIXED,
    PARTITION_PLAN, PaConfig, PaDecodeOpts, PaError, PaNormRope, PaPlanInfo, PaTensor, SCALE_NONE,
    SCALE_PER_TOKEN, SCALE_SCALAR, STATUS, check, desc, load, ref, stream_handle,
)

PAGE_SIZE = 128
HEAD_DIM = 128
GROUP_SIZE = 16
BLOCK_BYTES = PAGE_SIZE * HEAD_DIM


def pa_decode(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
              cu_seqlens_q, sparse_page_idx, scale_mode, out, stream=None):
    """Paged decode attention into ``out`` (see ``pa_decode`` in include/fp8pa.h)."""
    lib = load()
    d = [desc(t) for t in (q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                           cu_seqlens_q, sparse_page_idx)]
    do = desc(out)
    check(lib.pa_decode(*[ref(x) for x in d], int(scale_mode), ref(do), stream_handle(stream)))
    return out


def _decode_opts(sm_scale, max_q_len, force_parts, main_begin_event, main_end_event, prefetch_depth,
                 workgroup_waves, merge_mode, partition_mode):
    opts = PaDecodeOpts()
    opts.sm_scale = float(sm_scale)
    opts.max_q_len = int(max_q_len)
    opts.force_parts = int(force_parts)
    opts.prefetch_depth = int(prefetch_depth)
    opts.workgroup_waves = int(workgroup_waves)
    opts.merge_mode = int(merge_mode)
    opts.partition_mode = int(partition_mode)
    opts.main_begin_event = main_begin_event.cuda_event if main_begin_event is not None else None
    opts.main_end_event = main_end_event.cuda_event if main_end_event is not None else None
    return opts


def pa_decode_ex(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                 cu_seqlens_q, sparse_page_idx, scale_mode, out, sm_scale=0.0, max_q_len=0,
                 force_parts=0, main_begin_event=None, main_end_event=None, prefetch_depth=0,
                 workgroup_waves=0, merge_mode=0, partition_mode=0, stream=None):
    """``pa_decode`` with options; events are torch.cuda.Event objects that
    have been recorded once (so they exist)."""
    lib = load()
    opts = _decode_opts(sm_scale, max_q_len, force_parts, main_begin_event, main_end_event, prefetch_depth,
                        workgroup_waves, merge_mode, partition_mode)
    d = [desc(t) for t in (q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                           cu_seqlens_q, sparse_page_idx)]
    do = desc(out)
    check(lib.pa_decode_ex(*[ref(x) for x in d], int(scale_mode), ref(do), ctypes.byref(opts),
                           stream_handle(stream)))
    return out


def pa_decode_noalloc(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                      cu_seqlens_q, sparse_page_idx, scale_mode, out, sm_scale=0.0, max_q_len=0,
                      force_parts=0, main_begin_event=None, main_end_event=None, prefetch_depth=0,
                      workgroup_waves=0, merge_mode=0, partition_mode=0, stream=None):
    """``pa_decode_ex`` on the library's fixed scratch array: allocates
    nothing (see ``pa_decode_noalloc`` in include/fp8pa.h for its limit and
    why calls on one device must not overlap)."""
    lib = load()
    opts = _decode_opts(sm_scale, max_q_len, force_parts, main_begin_event, main_end_event, prefetch_depth,
                        workgroup_waves, merge_mode, partition_mode)
    d = [desc(t) for t in (q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                           cu_seqlens_q, sparse_page_idx)]
    do = desc(out)
    check(lib.pa_decode_noalloc(*[ref(x) for x in d], int(scale_mode), ref(do), ctypes.byref(opts),
                                stream_handle(stream)))
    return out


def pa_decode_write(q, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, block_table,
                    context_lens, cu_seqlens_q, scale_mode, out, sm_scale=0.0, max_q_len=0, force_parts=0,
                    main_begin_event=None, main_end_event=None, prefetch_depth=0, workgroup_waves=0,
                    merge_mode=0, partition_mode=0, sparse_page_idx=None, stream=None):
    """One decode step: ``kv_quant_write`` of the rows' own new tokens, then
    ``pa_decode_ex`` over the written cache (dense, or block-sparse with
    ``sparse_page_idx``), the write done inside the decode launch where it
    can be (see ``pa_decode_write`` in include/fp8pa.h)."""
    lib = load()
    opts = _decode_opts(sm_scale, max_q_len, force_parts, main_begin_event, main_end_event, prefetch_depth,
                        workgroup_waves, merge_mode, partition_mode)
    d = [desc(t) for t in (q, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, block_table,
                           context_lens, cu_seqlens_q, sparse_page_idx)]
    do = desc(out)
    check(lib.pa_decode_write(*[ref(x) for x in d], int(scale_mode), ref(do), ctypes.byref(opts),
                              stream_handle(stream)))
    return out


CHECK_KINDS = ("cu_ends", "cu_order", "ctx_short", "table_id", "sparse_id", "sparse_dup", "scale")


def pa_check_decode_inputs(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                           cu_seqlens_q, sparse_page_idx, scale_mode, out, report, stream=None):
    """Device-side check of a ``pa_decode`` call's inputs into ``report``
    (a device int32 tensor of 16 entries; see ``pa_check_decode_inputs`` in
    include/fp8pa.h).  Read ``report`` after synchronising the stream."""
    lib = load()
    if report.dtype != torch.int32 or report.numel() < 16 or not report.is_cuda:
        raise ValueError("report must be a device int32 tensor of at least 16 entries")
    d = [desc(t) for t in (q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                           cu_seqlens_q, sparse_page_idx)]
    do = desc(out)
    check(lib.pa_check_decode_inputs(*[ref(x) for x in d], int(scale_mode), ref(do), report.data_ptr(),
                                     stream_handle(stream)))
    return report


def check_report(report):
    """The report as a dict: violating items, the kinds found and the
    smallest offending index of each kind."""
    r = [int(x) for x in report.cpu().tolist()[:2 + len(CHECK_KINDS)]]
    return {"count": r[0],
            "kinds": [k for i, k in enumerate(CHECK_KINDS) if r[1] >> i & 1],
            "first": {k: r[2 + i] for i, k in enumerate(CHECK_KINDS) if r[1] >> i & 1}}


def kv_quant_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_mode,
                   stream=None):
    """Quantize and store new K/V tokens (see ``kv_quant_write`` in include/fp8pa.h)."""
    lib = load()
    d = [desc(t) for t in (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)]
    check(lib.kv_quant_write(*[ref(x) for x in d], int(scale_mode), stream_handle(stream)))


def kv_norm_rope_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, scale_mode,
                       positions, cos=None, sin=None, rotary_dim=0, neox=True, k_norm_weight=None,
                       q_norm_weight=None, eps=1e-6, weight_offset=0.0, q=None, q_out=None, stream=None):
    """``kv_quant_write`` fused with the key's RMS norm and rotary embedding,
    and the same transform of ``q`` into ``q_out`` (see ``kv_norm_rope_write``
    in include/fp8pa.h)."""
    lib = load()
    keep = [desc(t) for t in (positions, cos, sin, k_norm_weight, q_norm_weight)]
    nr = PaNormRope()
    nr.positions, nr.cos, nr.sin, nr.k_norm_weight, nr.q_norm_weight = [
        None if x is None else ctypes.pointer(x) for x in keep]
    nr.rotary_dim = int(rotary_dim)
    nr.neox = 1 if neox else 0
    nr.eps = float(eps)
    nr.weight_offset = float(weight_offset)
    d = [desc(t) for t in (q, q_out, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)]
    check(lib.kv_norm_rope_write(*[ref(x) for x in d], int(scale_mode), ctypes.byref(nr),
                                 stream_handle(stream)))
    return q_out


def pa_index_topk(q_idx, index_cache, block_table, context_lens, cu_seqlens_q, sparse_page_idx,
                  block_scores, sm_scale=0.0, max_q_len=0, stream=None):
    """Block scores and per-row top-k pages (see ``pa_index_topk`` in include/fp8pa.h)."""
    lib = load()
    d = [desc(t) for t in (q_idx, index_cache, block_table, context_lens, cu_seqlens_q)]
    ds, db = desc(sparse_page_idx), desc(block_scores)
    check(lib.pa_index_topk(*[ref(x) for x in d], int(max_q_len), float(sm_scale), ref(ds), ref(db),
                            stream_handle(stream)))
    return sparse_page_idx


def make_config(num_kv_heads, rows, batch, max_pages, topk=0, ragged=False, max_q_len=0,
                scale_mode=SCALE_PER_TOKEN, kv_dtype=1, force_parts=0, group_size=GROUP_SIZE,
                head_dim=HEAD_DIM, page_size=PAGE_SIZE, merge_mode=0, partition_mode=0):
    c = PaConfig()
    c.num_kv_heads, c.group_size, c.head_dim, c.page_size = num_kv_heads, group_size, head_dim, page_size
    c.kv_dtype, c.scale_mode = kv_dtype, scale_mode
    c.rows, c.batch, c.max_pages, c.topk = rows, batch, max_pages, topk
    c.ragged, c.max_q_len, c.force_parts = int(bool(ragged)), max_q_len, force_parts
    c.merge_mode = merge_mode
    c.partition_mode = partition_mode
    return c


def pa_query_support(cfg):
    """0 if the configuration is served, else the pa_status it would fail with."""
    return load().pa_query_support(ctypes.byref(cfg))


def pa_plan_describe(cfg):
    """The plan (as a dict) a configuration maps to; raises PaError if refused."""
    info = PaPlanInfo()
    check(load().pa_plan_describe(ctypes.byref(cfg), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in PaPlanInfo._fields_}


def pa_reserve(cfg, stream=None):
    check(load().pa_reserve(ctypes.byref(cfg), stream_handle(stream)))


def pa_release():
    check(load().pa_release())


def pa_last_error():
    return load().pa_last_error().decode()
