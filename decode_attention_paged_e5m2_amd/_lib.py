"""ctypes declarations for libxqa.so (mirrors include/xqa.h)."""

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libxqa.so")

XQA_OK = 0
XQA_ERR_INVALID_ARG = 1
XQA_ERR_UNSUPPORTED = 2
XQA_ERR_OUT_OF_MEMORY = 3
XQA_ERR_HIP = 4

EXPORTED = [
    "xqa_create", "xqa_destroy", "xqa_get_info", "xqa_decode", "xqa_decode_noalloc", "xqa_decode_multi",
    "xqa_decode_fp8", "xqa_decode_append", "xqa_decode_pages", "xqa_decode_split",
    "xqa_decode_combine", "xqa_append_kv", "xqa_plan", "xqa_debug_widen_e5m2",
    "xqa_debug_widen_e4m3", "xqa_status_string", "xqa_last_error",
]


class XqaConfig(ctypes.Structure):
    _fields_ = [
        ("max_batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_work_items", ctypes.c_int32),
        ("max_query_tokens", ctypes.c_int32),
        ("max_selected_pages", ctypes.c_int32),
    ]


class XqaInfo(ctypes.Structure):
    _fields_ = [
        ("device", ctypes.c_int32),
        ("max_work_items", ctypes.c_int32),
        ("items_per_head", ctypes.c_int32),
        ("token_granule", ctypes.c_int32),
        ("threads_per_item", ctypes.c_int32),
        ("item_stride_floats", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("kernels_per_step", ctypes.c_int32),
    ]


class XqaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_name(status)}: {detail}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library. Fails loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first "
            "(python -m decode_attention_paged_e5m2_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.xqa_create.argtypes = [ctypes.POINTER(XqaConfig), ctypes.POINTER(vp)]
    lib.xqa_destroy.argtypes = [vp]
    lib.xqa_get_info.argtypes = [vp, ctypes.POINTER(XqaInfo)]
    dec = [vp, vp, vp, vp, vp, vp, i32, f32, vp, vp]
    lib.xqa_decode.argtypes = dec
    lib.xqa_decode_noalloc.argtypes = [ctypes.POINTER(XqaConfig)] + dec[1:]
    lib.xqa_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp]
    lib.xqa_decode_fp8.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, f32, f32, f32,
                                   vp, vp]
    lib.xqa_decode_pages.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp]
    lib.xqa_decode_split.argtypes = dec
    lib.xqa_decode_combine.argtypes = [vp, vp, i32, vp, vp]
    lib.xqa_append_kv.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.xqa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp]
    lib.xqa_plan.argtypes = [vp, ctypes.POINTER(i32), i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.xqa_debug_widen_e5m2.argtypes = [vp, vp, vp, i64, vp]
    lib.xqa_debug_widen_e4m3.argtypes = [vp, vp, vp, i64, vp]
    lib.xqa_status_string.argtypes = [ctypes.c_int]
    lib.xqa_status_string.restype = ctypes.c_char_p
    lib.xqa_last_error.argtypes = []
    lib.xqa_last_error.restype = ctypes.c_char_p
    for name in ("xqa_create", "xqa_destroy", "xqa_get_info", "xqa_decode", "xqa_decode_noalloc",
                 "xqa_decode_multi",
                 "xqa_decode_fp8", "xqa_debug_widen_e4m3", "xqa_decode_append", "xqa_decode_pages",
                 "xqa_decode_split",
                 "xqa_decode_combine", "xqa_append_kv", "xqa_plan", "xqa_debug_widen_e5m2"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load().xqa_status_string(status).decode()


def check(status: int) -> None:
    if status != XQA_OK:
        raise XqaError(status, load().xqa_last_error().decode())
