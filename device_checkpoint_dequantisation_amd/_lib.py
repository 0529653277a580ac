"""ctypes declarations of libstmat.so's C ABI (include/stmat.h).  Loading fails loudly if the
library has not been built; there is no fallback implementation."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstmat.so")

ST_MAX_NDIM = 8
KINDS = ("PASS_BF16", "CAST_F16", "CAST_F32", "FP8_TENSOR", "FP8_BLOCK128", "NVFP4", "MXFP8", "MXFP4")
OUT_DTYPES = ("bf16", "f16", "f32")   # st_out_dtype codes 0, 1, 2
MAT_SLICES = 1
MAT_STREAM_STORES = 2        # st_materialize_as flag: non-temporal output stores
TABLE_STREAM_STORES = 1      # st_table_header.flags: outputs larger than the last-level cache
DTYPES = ("BOOL", "U8", "I8", "F8_E4M3", "F8_E5M2", "F8_E8M0", "I16", "U16", "F16", "BF16", "I32", "U32", "F32",
          "I64", "U64", "F64", "F4", "F6_E2M3", "F6_E3M2")
STATUS = {0: "ST_OK", -1: "ST_E_ARG", -2: "ST_E_IO", -3: "ST_E_HEADER", -4: "ST_E_JSON", -5: "ST_E_DTYPE",
          -6: "ST_E_SHAPE", -7: "ST_E_OFFSETS", -8: "ST_E_SCALE", -9: "ST_E_NOMEM", -10: "ST_E_HIP"}


class TensorMeta(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * ST_MAX_NDIM), ("begin", C.c_uint64), ("end", C.c_uint64)]


class OutputInfo(C.Structure):
    _fields_ = [("name", C.c_char_p), ("kind", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * ST_MAX_NDIM), ("numel", C.c_uint64), ("tensor", C.c_int64),
                ("scale", C.c_int64), ("scale2", C.c_int64)]


class Desc(C.Structure):
    _fields_ = [("src", C.c_uint64), ("scale", C.c_uint64), ("scale2", C.c_uint64), ("pitch", C.c_uint32),
                ("flags", C.c_uint32),
                ("unit_begin", C.c_uint32), ("unit_end", C.c_uint32), ("tail", C.c_uint32), ("out", C.c_uint32),
                ("cols", C.c_uint32), ("grid_cols", C.c_uint32), ("div_magic", C.c_uint32), ("meta", C.c_uint32)]


assert C.sizeof(Desc) == 64


class TableHeader(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("n_desc", C.c_uint32), ("units", C.c_uint64), ("desc_offset", C.c_uint64),
                ("map_offset", C.c_uint64), ("bytes", C.c_uint64), ("out_dtype", C.c_uint32), ("flags", C.c_uint32),
                ("reserved", C.c_uint64 * 2)]


assert C.sizeof(TableHeader) == 64
TABLE_MAGIC = 0x334D5453
UNITS_PER_GROUP = 4
NOALLOC_SCRATCH_BYTES = 32 << 20


DESC_EXACT = 1
DESC_SPLIT = 2


class Slice(C.Structure):
    _fields_ = [("output", C.c_uint32), ("reserved", C.c_uint32), ("row_begin", C.c_int64), ("row_end", C.c_int64),
                ("col_begin", C.c_int64), ("col_end", C.c_int64)]


assert C.sizeof(Slice) == 40


class PlanOpts(C.Structure):
    _fields_ = [("unit_log2_scale", C.c_uint32), ("flags", C.c_uint32)]


class StreamRange(C.Structure):
    _fields_ = [("begin", C.c_uint64), ("end", C.c_uint64), ("dst", C.c_uint64), ("step", C.c_uint32),
                ("reserved", C.c_uint32)]


PLAN_PACK = 1


class StreamStep(C.Structure):
    _fields_ = [("bytes", C.c_uint64), ("first_range", C.c_uint32), ("n_ranges", C.c_uint32),
                ("first_out", C.c_uint32), ("n_out", C.c_uint32), ("table_offset", C.c_uint64), ("units", C.c_uint64)]


class StreamStats(C.Structure):
    _fields_ = [("seconds_read", C.c_double), ("seconds_wait", C.c_double), ("bytes_read", C.c_uint64),
                ("steps", C.c_uint32), ("launches", C.c_uint32), ("seconds_first_launch", C.c_double)]


assert C.sizeof(StreamRange) == 32 and C.sizeof(StreamStep) == 40 and C.sizeof(StreamStats) == 40


# name -> (restype, argtypes); the full list of exported symbols the header declares.
SIGNATURES = {
    "st_last_error": (C.c_char_p, []),
    "st_header_size": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint64)]),
    "st_index_build": (C.c_int, [C.c_void_p, C.c_uint64, C.c_uint64, C.POINTER(PlanOpts), C.POINTER(C.c_void_p)]),
    "st_index_open": (C.c_int, [C.c_char_p, C.POINTER(PlanOpts), C.POINTER(C.c_void_p)]),
    "st_index_free": (None, [C.c_void_p]),
    "st_index_data_offset": (C.c_uint64, [C.c_void_p]),
    "st_index_data_size": (C.c_uint64, [C.c_void_p]),
    "st_index_blob_bytes": (C.c_uint64, [C.c_void_p]),
    "st_index_count": (C.c_size_t, [C.c_void_p]),
    "st_index_tensor": (C.c_int, [C.c_void_p, C.c_size_t, C.POINTER(TensorMeta)]),
    "st_index_find": (C.c_int64, [C.c_void_p, C.c_char_p]),
    "st_index_metadata_json": (C.c_char_p, [C.c_void_p]),
    "st_index_num_outputs": (C.c_size_t, [C.c_void_p]),
    "st_index_output": (C.c_int, [C.c_void_p, C.c_size_t, C.POINTER(OutputInfo)]),
    "st_index_output_offset": (C.c_uint64, [C.c_void_p, C.c_size_t]),
    "st_index_output_arena_bytes": (C.c_uint64, [C.c_void_p]),
    "st_index_traffic_bytes": (C.c_uint64, [C.c_void_p]),
    "st_index_device_bytes": (C.c_uint64, [C.c_void_p]),
    "st_index_table": (C.c_void_p, [C.c_void_p, C.POINTER(C.c_size_t), C.POINTER(C.c_uint64)]),
    "st_index_descs": (C.c_void_p, [C.c_void_p, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "st_index_table_subset": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint32), C.c_size_t, C.c_void_p, C.c_size_t,
                                        C.POINTER(C.c_size_t), C.POINTER(C.c_uint64)]),
    "st_index_table_slices": (C.c_int, [C.c_void_p, C.POINTER(Slice), C.c_size_t, C.c_void_p, C.c_size_t,
                                        C.POINTER(C.c_size_t), C.POINTER(C.c_uint64)]),
    "st_index_slice_numel": (C.c_int, [C.c_void_p, C.POINTER(Slice), C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
    "st_stage_file": (C.c_int, [C.c_char_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p,
                                C.POINTER(C.c_double)]),
    "st_materialize": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]),
    "st_materialize_slices": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]),
    "st_materialize_as": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p, C.c_uint32, C.c_uint32,
                                    C.c_void_p]),
    "st_materialize_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_size_t, C.c_void_p, C.c_size_t,
                                         C.c_uint32, C.c_uint32, C.c_void_p]),
    "st_index_out_dtype": (C.c_uint32, [C.c_void_p]),
    "st_stream_plan_build": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(C.c_void_p)]),
    "st_stream_plan_select": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint32), C.c_size_t, C.c_uint64, C.c_uint32,
                                        C.POINTER(C.c_void_p)]),
    "st_stream_plan_free": (None, [C.c_void_p]),
    "st_stream_plan_blob_bytes": (C.c_uint64, [C.c_void_p]),
    "st_read_plan": (C.c_int, [C.c_char_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.POINTER(C.c_double)]),
    "st_read_plans": (C.c_int, [C.c_char_p, C.c_void_p, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
                                C.POINTER(C.c_size_t), C.c_size_t, C.POINTER(C.c_double)]),
    "st_stream_plan_chunk_bytes": (C.c_uint64, [C.c_void_p]),
    "st_stream_plan_num_steps": (C.c_size_t, [C.c_void_p]),
    "st_stream_plan_step": (C.c_int, [C.c_void_p, C.c_size_t, C.POINTER(StreamStep)]),
    "st_stream_plan_ranges": (C.POINTER(StreamRange), [C.c_void_p, C.POINTER(C.c_size_t)]),
    "st_stream_plan_order": (C.POINTER(C.c_uint32), [C.c_void_p, C.POINTER(C.c_size_t)]),
    "st_stream_plan_tables": (C.c_void_p, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "st_stream_file": (C.c_int, [C.c_char_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_size_t, C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(StreamStats)]),
}

_lib = None


def lib():
    """The loaded library; raises if it is missing (build it with __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libstmat.so is not built at {LIB_PATH}; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class StError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().st_last_error().decode("utf-8", "replace")
        super().__init__(f"{where}: {STATUS.get(code, code)}: {msg}")
        self.code = code


def check(code: int, where: str):
    if code != 0:
        raise StError(code, where)
