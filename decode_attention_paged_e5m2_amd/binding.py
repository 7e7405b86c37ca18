"""Thin Python binding over libxqa.so: argument checks and marshalling only.

PyTorch provides device memory and the current HIP stream; every step of the
computation runs in the library's kernels. Optional arguments are keywords.
"""

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

HEAD_DIM = 128
PAGE_SIZE = 16


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream: Optional[torch.cuda.Stream], device: torch.device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


_KV_FORMATS = {"e5m2": 0, "e4m3": 1}   # xqa_kv_format_t


class Xqa:
    """A decode-attention handle: fixed head counts, capacity and workspace.

    Example::

        xqa = Xqa(max_batch=16, num_q_heads=32, num_kv_heads=4, max_pages_per_seq=16384)
        out = xqa.decode(q=q, k_pages=k, v_pages=v, block_table=bt,
                         context_lens=lens, scale=1 / 128 ** 0.5)
    """

    def __init__(self, *, max_batch: int, num_q_heads: int, num_kv_heads: int,
                 max_pages_per_seq: int, head_dim: int = HEAD_DIM, page_size: int = PAGE_SIZE,
                 max_work_items: int = 0, max_query_tokens: int = 1,
                 max_selected_pages: int = 0, device: Optional[torch.device] = None):
        lib = _lib.load()
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        cfg = _lib.XqaConfig(max_batch, num_q_heads, num_kv_heads, head_dim, page_size,
                             max_pages_per_seq, max_work_items, max_query_tokens,
                             max_selected_pages)
        handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _lib.check(lib.xqa_create(ctypes.byref(cfg), ctypes.byref(handle)))
        self._h = handle
        self.max_batch = max_batch
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.max_pages_per_seq = max_pages_per_seq
        self.max_query_tokens = max_query_tokens
        self.max_selected_pages = max_selected_pages
        self.head_dim = head_dim
        self.page_size = page_size

    # ----------------------------------------------------------------- info
    @property
    def info(self) -> dict:
        inf = _lib.XqaInfo()
        _lib.check(_lib.load().xqa_get_info(self._h, ctypes.byref(inf)))
        return {k: getattr(inf, k) for k, _ in _lib.XqaInfo._fields_}

    def plan(self, context_lens) -> Tuple[int, int]:
        """Host mirror of the device plan: (split length in tokens, work items)."""
        lens = [int(x) for x in (context_lens.tolist() if hasattr(context_lens, "tolist")
                                 else context_lens)]
        arr = (ctypes.c_int32 * len(lens))(*lens)
        S, items = ctypes.c_int32(), ctypes.c_int32()
        _lib.check(_lib.load().xqa_plan(self._h, arr, len(lens), ctypes.byref(S), ctypes.byref(items)))
        return S.value, items.value

    # ------------------------------------------------------------ checking
    def _check(self, q, k_pages, v_pages, block_table, context_lens, out, batch):
        dev = self.device
        for name, t, dt in (("q", q, torch.float16), ("k_pages", k_pages, torch.uint8),
                            ("v_pages", v_pages, torch.uint8), ("block_table", block_table, torch.int32),
                            ("context_lens", context_lens, torch.int32), ("out", out, torch.float16)):
            _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
            _need(t.dtype == dt, f"{name} must be {dt}, got {t.dtype}")
            _need(t.device == dev, f"{name} must be on {dev}, got {t.device}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
        Hq, Hkv, D, P = self.num_q_heads, self.num_kv_heads, self.head_dim, self.page_size
        if q.dim() == 4:   # [batch, M, Hq, D]: several query tokens per sequence
            _need(q.shape[2:] == (Hq, D) and q.shape[0] >= batch
                  and 1 <= q.shape[1] <= self.max_query_tokens,
                  f"q must be [>= batch, 1..{self.max_query_tokens}, {Hq}, {D}], got {tuple(q.shape)}")
            _need(out.dim() == 4 and out.shape[1:] == q.shape[1:] and out.shape[0] >= batch,
                  f"out must be [>= batch, {q.shape[1]}, {Hq}, {D}], got {tuple(out.shape)}")
        else:
            _need(q.dim() == 3 and q.shape[1:] == (Hq, D) and q.shape[0] >= batch,
                  f"q must be [>= batch, {Hq}, {D}], got {tuple(q.shape)}")
            _need(out.dim() == 3 and out.shape[1:] == (Hq, D) and out.shape[0] >= batch,
                  f"out must be [>= batch, {Hq}, {D}], got {tuple(out.shape)}")
        _need(k_pages.dim() == 4 and k_pages.shape[1:] == (Hkv, P, D),
              f"k_pages must be [num_pages, {Hkv}, {P}, {D}], got {tuple(k_pages.shape)}")
        _need(v_pages.shape == k_pages.shape, "v_pages must have k_pages' shape")
        _need(block_table.dim() == 2 and block_table.shape[1] == self.max_pages_per_seq
              and block_table.shape[0] >= batch,
              f"block_table must be [>= batch, {self.max_pages_per_seq}], got {tuple(block_table.shape)}")
        _need(context_lens.dim() == 1 and context_lens.shape[0] >= batch,
              "context_lens must be [>= batch]")
        _need(1 <= batch <= self.max_batch, f"batch must be in [1, {self.max_batch}]")

    def _args(self, q, k_pages, v_pages, block_table, context_lens, out, batch, scale, stream):
        if batch is None:
            batch = q.shape[0]
        if out is None:
            out = torch.empty_like(q)
        self._check(q, k_pages, v_pages, block_table, context_lens, out, batch)
        scale = float(scale)
        _need(math.isfinite(scale), "scale must be finite")
        return out, (self._h, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                     _ptr(context_lens), int(batch), ctypes.c_float(scale), _ptr(out),
                     _stream_ptr(stream, self.device))

    # -------------------------------------------------------------- decode
    def decode(self, *, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
               block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
               out: Optional[torch.Tensor] = None, batch: Optional[int] = None,
               kv_format: str = "e5m2", k_scale: float = 1.0, v_scale: float = 1.0,
               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """One decode step (split kernel + combine kernel) on the current stream.

        q is [B, Hq, D] (one new token per sequence, xqa_decode) or
        [B, M, Hq, D] (M new tokens, causal among themselves,
        xqa_decode_multi); out has q's shape. kv_format "e4m3" or scales
        other than 1 go through xqa_decode_fp8."""
        _need(kv_format in _KV_FORMATS, f"kv_format must be one of {sorted(_KV_FORMATS)}")
        out, args = self._args(q, k_pages, v_pages, block_table, context_lens, out, batch, scale, stream)
        M = int(q.shape[1]) if q.dim() == 4 else 1
        lib = _lib.load()
        if kv_format != "e5m2" or k_scale != 1.0 or v_scale != 1.0:
            _need(math.isfinite(k_scale) and math.isfinite(v_scale), "scales must be finite")
            _lib.check(lib.xqa_decode_fp8(args[0], _KV_FORMATS[kv_format], *args[1:7], M, args[7],
                                          ctypes.c_float(k_scale), ctypes.c_float(v_scale),
                                          *args[8:]))
        elif q.dim() == 4:
            _lib.check(lib.xqa_decode_multi(*args[:7], M, *args[7:]))
        else:
            _lib.check(lib.xqa_decode(*args))
        return out

    def decode_pages(self, *, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                     block_table: torch.Tensor, context_lens: torch.Tensor,
                     page_select: torch.Tensor, select_counts: torch.Tensor, scale: float,
                     out: Optional[torch.Tensor] = None, batch: Optional[int] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Decode over a selected subset of each sequence's pages
        (xqa_decode_pages): page_select int32 [B, S] holds ascending logical
        page indices, select_counts int32 [B] how many of each row to use;
        q is [B, Hq, D]. The handle needs max_selected_pages >= S."""
        _need(isinstance(q, torch.Tensor) and q.dim() == 3, "decode_pages() takes q [B, Hq, D]")
        out, args = self._args(q, k_pages, v_pages, block_table, context_lens, out, batch, scale, stream)
        batch = int(args[6])
        for name, t in (("page_select", page_select), ("select_counts", select_counts)):
            _need(isinstance(t, torch.Tensor) and t.dtype == torch.int32 and t.device == self.device
                  and t.is_contiguous(), f"{name} must be contiguous int32 on {self.device}")
        _need(page_select.dim() == 2 and page_select.shape[0] >= batch
              and 1 <= page_select.shape[1] <= self.max_selected_pages,
              f"page_select must be [>= batch, 1..{self.max_selected_pages}], "
              f"got {tuple(page_select.shape)}")
        _need(select_counts.dim() == 1 and select_counts.shape[0] >= batch,
              "select_counts must be [>= batch]")
        h, qp, kp, vp, btp, clp, b, sc, op, st = args
        _lib.check(_lib.load().xqa_decode_pages(h, qp, kp, vp, btp, clp, _ptr(page_select),
                                                _ptr(select_counts), int(page_select.shape[1]),
                                                b, sc, op, st))
        return out

    def split(self, *, q, k_pages, v_pages, block_table, context_lens, scale, out=None,
              batch=None, stream=None) -> torch.Tensor:
        """First stage only (xqa_decode_split, one query token); combine() must follow."""
        _need(isinstance(q, torch.Tensor) and q.dim() == 3, "split() takes q [B, Hq, D]")
        out, args = self._args(q, k_pages, v_pages, block_table, context_lens, out, batch, scale, stream)
        _lib.check(_lib.load().xqa_decode_split(*args))
        return out

    def combine(self, *, context_lens, out, batch=None, stream=None) -> torch.Tensor:
        """Second stage only (xqa_decode_combine)."""
        if batch is None:
            batch = out.shape[0]
        _need(isinstance(context_lens, torch.Tensor) and context_lens.dtype == torch.int32
              and context_lens.device == self.device and context_lens.is_contiguous(),
              "context_lens must be contiguous int32 on the handle's device")
        _need(isinstance(out, torch.Tensor) and out.dtype == torch.float16
              and out.device == self.device and out.is_contiguous(),
              "out must be contiguous float16 on the handle's device")
        _need(out.dim() == 3 and out.shape[1:] == (self.num_q_heads, self.head_dim)
              and out.shape[0] >= batch and context_lens.shape[0] >= batch
              and 1 <= batch <= self.max_batch, "bad shapes or batch")
        _lib.check(_lib.load().xqa_decode_combine(self._h, _ptr(context_lens), int(batch), _ptr(out),
                                                  _stream_ptr(stream, self.device)))
        return out

    def append_kv(self, *, k_new: torch.Tensor, v_new: torch.Tensor, block_table: torch.Tensor,
                  context_lens: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                  batch: Optional[int] = None, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Write each sequence's new token (k_new, v_new: float16 [B, Hkv, 128]) into the
        pages as E5M2 (xqa_append_kv); context_lens counts the new token."""
        dev = self.device
        if batch is None:
            batch = k_new.shape[0] if isinstance(k_new, torch.Tensor) else 0
        for name, t, dt in (("k_new", k_new, torch.float16), ("v_new", v_new, torch.float16),
                            ("block_table", block_table, torch.int32),
                            ("context_lens", context_lens, torch.int32),
                            ("k_pages", k_pages, torch.uint8), ("v_pages", v_pages, torch.uint8)):
            _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
            _need(t.dtype == dt, f"{name} must be {dt}")
            _need(t.device == dev, f"{name} must be on {dev}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
        H, D, P = self.num_kv_heads, self.head_dim, self.page_size
        _need(1 <= batch <= self.max_batch, "batch outside [1, max_batch]")
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            _need(t.dim() == 3 and t.shape[0] >= batch and t.shape[1:] == (H, D),
                  f"{name} must be [>= batch, {H}, {D}]")
        for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
            _need(t.dim() == 4 and t.shape[1:] == (H, P, D), f"{name} must be [pages, {H}, {P}, {D}]")
        _need(block_table.dim() == 2 and block_table.shape[0] >= batch
              and block_table.shape[1] == self.max_pages_per_seq,
              "block_table must be [>= batch, max_pages_per_seq]")
        _need(context_lens.dim() == 1 and context_lens.shape[0] >= batch,
              "context_lens must be [>= batch]")
        _lib.check(_lib.load().xqa_append_kv(self._h, _ptr(k_new), _ptr(v_new), _ptr(block_table),
                                             _ptr(context_lens), int(batch), _ptr(k_pages),
                                             _ptr(v_pages), _stream_ptr(stream, dev)))

    def decode_append(self, *, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                      context_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                      batch: Optional[int] = None,
                      stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """append_kv + decode in one call (xqa_decode_append): the new token's
        rows are written into the pages and attended to; q is [B, Hq, D]."""
        _need(isinstance(q, torch.Tensor) and q.dim() == 3, "decode_append() takes q [B, Hq, D]")
        out, args = self._args(q, k_pages, v_pages, block_table, context_lens, out, batch, scale, stream)
        batch = int(args[6])
        H, D = self.num_kv_heads, self.head_dim
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            _need(isinstance(t, torch.Tensor) and t.dtype == torch.float16 and t.device == self.device
                  and t.is_contiguous(), f"{name} must be contiguous float16 on {self.device}")
            _need(t.dim() == 3 and t.shape[0] >= batch and t.shape[1:] == (H, D),
                  f"{name} must be [>= batch, {H}, {D}]")
        h, qp, kp, vp, btp, clp, b, sc, op, st = args
        _lib.check(_lib.load().xqa_decode_append(h, qp, _ptr(k_new), _ptr(v_new), kp, vp, btp, clp,
                                                 b, sc, op, st))
        return out

    # ----------------------------------------------------------- lifetime
    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            _lib.check(_lib.load().xqa_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _debug_widen(fn, codes, stream):
    _need(codes.dtype == torch.uint8 and codes.is_cuda and codes.is_contiguous(),
          "codes must be a contiguous uint8 GPU tensor")
    bits = torch.empty(codes.shape, dtype=torch.int16, device=codes.device)
    vals = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _lib.check(fn(_ptr(codes), _ptr(bits), _ptr(vals), codes.numel(),
                  _stream_ptr(stream, codes.device)))
    return bits, vals


def debug_widen_e5m2(codes: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
    """Widen uint8 E5M2 codes on the GPU with the kernels' own routine.

    Returns (binary16 bit patterns as int16, values as float32).
    """
    return _debug_widen(_lib.load().xqa_debug_widen_e5m2, codes, stream)


def debug_widen_e4m3(codes: torch.Tensor, stream: Optional[torch.cuda.Stream] = None):
    """Widen uint8 E4M3 codes on the GPU with the kernels' own routine."""
    return _debug_widen(_lib.load().xqa_debug_widen_e4m3, codes, stream)
