"""CPU oracle for paged FP8-E5M2 grouped-query decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library under
``decode_attention_paged_e5m2_amd/`` and its Python binding) imports, links or
calls this package. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.

What it computes, and where that comes from:

* The page "[Kernel][SM70] Pipeline batched E5M2 XQA decode" (sections Purpose
  and Starting bottleneck) names the operation: batched decode attention in
  which each sequence's one new query token attends over a long, ragged,
  paged KV cache whose K and V are stored as FP8 E5M2, with query heads
  sharing KV heads (XQA, i.e. grouped-query attention). Its section "Pending
  work and gates" lists the phases K load + E5M2 conversion, QK, V load +
  conversion and PV, and asks for randomized physical pages.
* The pages print no formula, no bit layout and no worked example. The
  oracle therefore writes out the plain definition of scaled-dot-product
  attention for one query token (softmax over all cached tokens, then the
  probability-weighted sum of V), and decodes E5M2 with the closed form of
  the OCP 8-bit floating-point E5M2 format. Every reading taken where the
  pages are silent is listed in the design notes; the ones this code relies
  on are repeated in the docstrings below.

All arithmetic is float64 numpy. Functions:

* ``e5m2.decode_e5m2``          closed-form E5M2 code -> float64
* ``attention.decode_attention``  the full batched operation (float64 output)
* ``attention.decode_attention_row``  one (sequence, query head) row
* ``attention.decode_attention_multi``  M new query tokens per sequence,
  causal among themselves
* ``e4m3.decode_e4m3``          closed-form OCP E4M3 code -> float64
* ``attention.decode_attention_fp8``  the operation over an E5M2 or E4M3
  cache with per-tensor K and V dequantisation scales
* ``attention.partial_state`` / ``attention.merge_states``  the split-context
  form (running max, sum of weights, unnormalised output) and its
  log-sum-exp merge, used to pin the split-K + combine arithmetic.
* ``append.encode_e5m2``        float -> E5M2 code, nearest finite value with
  ties to even (the KV append's rounding)
* ``append.append_kv``          the KV append: each sequence's new token
  encoded and written to its page slot
* ``pages.decode_attention_pages``  attention over a selected subset of each
  sequence's pages (``pages.kept_pages`` / ``pages.selected_tokens`` give the
  pages and tokens a selection keeps)

Pins (tests marked ``not gpu``): all 256 codes against the IEEE binary16 view
of the code shifted into the high byte; single-token, constant-V, uniform-K,
zero-scale and shift-invariance special cases; page re-permutation; a
pure-Python brute force on tiny shapes; split-and-merge equals single pass.
"""

from .e5m2 import decode_e5m2, E5M2_TABLE, E5M2_MAX_FINITE
from .e4m3 import decode_e4m3, E4M3_TABLE, E4M3_MAX_FINITE
from .append import encode_e5m2, append_kv
from .pages import decode_attention_pages, kept_pages, selected_tokens
from .attention import (
    decode_attention,
    decode_attention_fp8,
    decode_attention_multi,
    decode_attention_row,
    gather_tokens,
    partial_state,
    merge_states,
)

__all__ = [
    "decode_e5m2",
    "E5M2_TABLE",
    "E5M2_MAX_FINITE",
    "decode_attention",
    "decode_attention_row",
    "decode_attention_multi",
    "gather_tokens",
    "partial_state",
    "merge_states",
    "encode_e5m2",
    "append_kv",
    "decode_e4m3",
    "E4M3_TABLE",
    "E4M3_MAX_FINITE",
    "decode_attention_fp8",
    "decode_attention_pages",
    "kept_pages",
    "selected_tokens",
]
