"""ctypes binding to libfp8pa.so: argument marshalling only.

Torch tensors are turned into ``pa_tensor`` descriptors (pointer, dtype,
shape, strides); every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing, loading fails.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FP8PA_LIB") or os.path.join(HERE, "libfp8pa.so")

MAX_DIMS = 6

DTYPE_U8, DTYPE_F8E4M3, DTYPE_BF16, DTYPE_F32, DTYPE_I32, DTYPE_I64 = 1, 2, 3, 4, 5, 6
SCALE_NONE, SCALE_SCALAR, SCALE_PER_TOKEN = 0, 1, 2
MERGE_PLAN, MERGE_SEPARATE, MERGE_IN_KERNEL = 0, 1, 2
PARTITION_PLAN, PARTITION_FIXED, PARTITION_BALANCED = 0, 1, 2

STATUS = {
    0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_DTYPE", -3: "PA_ERR_SHAPE",
    -4: "PA_ERR_LAYOUT", -5: "PA_ERR_UNSUPPORTED", -6: "PA_ERR_CAPACITY",
    -7: "PA_ERR_NOT_RESERVED", -8: "PA_ERR_HIP",
}

_TORCH_DTYPES = {
    torch.uint8: DTYPE_U8,
    torch.float8_e4m3fn: DTYPE_F8E4M3,
    torch.bfloat16: DTYPE_BF16,
    torch.float32: DTYPE_F32,
    torch.int32: DTYPE_I32,
    torch.int64: DTYPE_I64,
}


class PaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * MAX_DIMS),
        ("stride", ctypes.c_int64 * MAX_DIMS),
    ]


class PaNormRope(ctypes.Structure):
    _fields_ = [
        ("positions", ctypes.POINTER(PaTensor)),
        ("cos", ctypes.POINTER(PaTensor)),
        ("sin", ctypes.POINTER(PaTensor)),
        ("rotary_dim", ctypes.c_int32),
        ("neox", ctypes.c_int32),
        ("k_norm_weight", ctypes.POINTER(PaTensor)),
        ("q_norm_weight", ctypes.POINTER(PaTensor)),
        ("eps", ctypes.c_float),
        ("weight_offset", ctypes.c_float),
    ]


class PaDecodeOpts(ctypes.Structure):
    _fields_ = [
        ("sm_scale", ctypes.c_float),
        ("max_q_len", ctypes.c_int32),
        ("force_parts", ctypes.c_int32),
        ("main_begin_event", ctypes.c_void_p),
        ("main_end_event", ctypes.c_void_p),
        ("prefetch_depth", ctypes.c_int32),
        ("workgroup_waves", ctypes.c_int32),
        ("merge_mode", ctypes.c_int32),
        ("partition_mode", ctypes.c_int32),
    ]


class PaConfig(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("max_pages", ctypes.c_int64),
        ("topk", ctypes.c_int64),
        ("ragged", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("force_parts", ctypes.c_int32),
        ("merge_mode", ctypes.c_int32),
        ("partition_mode", ctypes.c_int32),
    ]


class PaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("rows_per_group", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("parts", ctypes.c_int32),
        ("pages_per_part", ctypes.c_int32),
        ("units", ctypes.c_int64),
        ("grid_x", ctypes.c_int64),
        ("grid_y", ctypes.c_int64),
        ("rows_bucket", ctypes.c_int64),
        ("pages_bucket", ctypes.c_int64),
        ("scratch_bytes", ctypes.c_int64),
        ("merge", ctypes.c_int32),
        ("merge_in_kernel", ctypes.c_int32),
        ("balanced", ctypes.c_int32),
    ]


EXPORTS = ("pa_decode", "pa_decode_ex", "pa_decode_noalloc", "pa_decode_write", "pa_check_decode_inputs", "kv_quant_write",
           "kv_norm_rope_write", "pa_index_topk", "pa_query_support", "pa_plan_describe", "pa_reserve", "pa_release", "pa_last_error")

_lib = None


def load():
    """Load libfp8pa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp8_paged_kv_pa_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    T = P(PaTensor)
    lib.pa_decode.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int, T, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_ex.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int, T, P(PaDecodeOpts), vp]
    lib.pa_decode_ex.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int, T, P(PaDecodeOpts), vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_write.argtypes = [T, T, T, T, T, T, T, T, T, T, T, T, ctypes.c_int, T, P(PaDecodeOpts), vp]
    lib.pa_decode_write.restype = ctypes.c_int
    lib.pa_check_decode_inputs.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int, T, vp, vp]
    lib.pa_check_decode_inputs.restype = ctypes.c_int
    lib.kv_quant_write.argtypes = [T, T, T, T, T, T, T, ctypes.c_int, vp]
    lib.kv_quant_write.restype = ctypes.c_int
    lib.kv_norm_rope_write.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int, P(PaNormRope), vp]
    lib.kv_norm_rope_write.restype = ctypes.c_int
    lib.pa_index_topk.argtypes = [T, T, T, T, T, ctypes.c_int, ctypes.c_float, T, T, vp]
    lib.pa_index_topk.restype = ctypes.c_int
    lib.pa_query_support.argtypes = [P(PaConfig)]
    lib.pa_query_support.restype = ctypes.c_int
    lib.pa_plan_describe.argtypes = [P(PaConfig), P(PaPlanInfo)]
    lib.pa_plan_describe.restype = ctypes.c_int
    lib.pa_reserve.argtypes = [P(PaConfig), vp]
    lib.pa_reserve.restype = ctypes.c_int
    lib.pa_release.argtypes = []
    lib.pa_release.restype = ctypes.c_int
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


class PaError(RuntimeError):
    def __init__(self, status, msg):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {msg}")


def check(status):
    if status != 0:
        raise PaError(status, load().pa_last_error().decode())
    return status


def desc(t):
    """pa_tensor descriptor of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if t.dtype not in _TORCH_DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > MAX_DIMS:
        raise ValueError("too many dimensions")
    d = PaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _TORCH_DTYPES[t.dtype]
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = s
        d.stride[i] = st
    return d


def ref(d):
    return None if d is None else ctypes.byref(d)


def stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream
