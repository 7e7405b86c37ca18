"""Paged FP8-E5M2 grouped-query decode attention on AMD MI355X (gfx950).

The computation lives in libxqa.so (hand-written HIP kernels behind the C ABI
declared in include/xqa.h); this package loads it and marshals arguments.
"""

from ._lib import LIB_PATH, XqaError, load as load_library
from .binding import Xqa, debug_widen_e4m3, debug_widen_e5m2

__all__ = ["Xqa", "debug_widen_e5m2", "debug_widen_e4m3", "XqaError", "load_library", "LIB_PATH"]
