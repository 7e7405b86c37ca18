"""KV append in the oracle: E5M2 encoding and the page scatter (test
infrastructure only).

The pages ("[Kernel][SM70] Pipeline batched E5M2 XQA decode", section
Purpose) deploy an FP8 E5M2 KV cache, so every decode step first stores the
new token's K and V as E5M2 bytes in the sequence's current page. They do
not spell out the rounding or the placement. Readings taken:

* Encoding: the nearest finite E5M2 value, ties to the code with the even
  mantissa (round to nearest even). Finite inputs beyond the largest
  magnitude, and infinities, therefore give +-57344 (saturation: the nearest
  finite value). The sign is kept, so negative values that round to zero
  give -0 (code 0x80). NaN gives code 0x7F with the input's sign bit.
* Placement: context_lens[b] = n already counts the new token, which is
  token n - 1 and goes to page block_table[b][(n - 1) // 16], slot
  (n - 1) % 16, for every KV head. A sequence with n <= 0, or whose token
  n - 1 lies beyond the block table's capacity, gets no write.
"""

import numpy as np

from .e5m2 import E5M2_TABLE

# Non-negative finite codes 0x00..0x7B decode to strictly increasing values.
_POS_CODES = np.arange(0x7C)
_POS_VALUES = E5M2_TABLE[:0x7C]


def encode_e5m2(x) -> np.ndarray:
    """Encode floats to E5M2 codes (uint8) by the nearest-value rule above."""
    v = np.asarray(x, dtype=np.float64)
    mag = np.abs(v)
    nan = np.isnan(v)
    mag = np.where(nan, 0.0, mag)
    # Neighbouring finite values below and above |x| (inf lies above all).
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(mag - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - mag)
    even_hi = (_POS_CODES[hi] % 2) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & even_hi)
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo])
    # At or past the largest finite value that value is the nearest one
    # (the distances above would lose it to rounding for huge inputs).
    code = np.where(mag >= _POS_VALUES[-1], 0x7B, code)
    code = np.where(nan, 0x7F, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def append_kv(k_pages, v_pages, block_table, context_lens, k_new, v_new):
    """Return copies of the K and V pools with each sequence's new token written.

    k_pages, v_pages: uint8 [num_pages, Hkv, P, D]; block_table: int [B, max_pages];
    context_lens: int [B] (lengths after the append); k_new, v_new: float [B, Hkv, D].
    """
    kp = np.array(k_pages, copy=True)
    vp = np.array(v_pages, copy=True)
    bt = np.asarray(block_table)
    lens = np.asarray(context_lens)
    page = kp.shape[2]
    capacity = bt.shape[1] * page
    kn = np.asarray(k_new)
    vn = np.asarray(v_new)
    for b in range(lens.shape[0]):
        n = int(lens[b])
        if n <= 0 or n > capacity:
            continue
        t = n - 1
        pg = int(bt[b, t // page])
        kp[pg, :, t % page, :] = encode_e5m2(kn[b])
        vp[pg, :, t % page, :] = encode_e5m2(vn[b])
    return kp, vp
