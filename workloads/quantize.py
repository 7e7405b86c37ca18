"""Round float32 draws to FP8 E5M2 bytes for synthetic K/V data.

Encoding: OCP 8-bit floating point E5M2 (sign, 5-bit exponent with bias 15,
2-bit mantissa, subnormals below 2^-14). Rounding: to nearest, ties to the
even code, computed directly from the float32 value (never through float16,
which would round twice). Magnitudes above the largest finite value 57344 are
clamped to it first (saturating), so the generator never emits inf or NaN.
A negative input that rounds to zero gives the negative-zero code 0x80.

Two implementations of the same rounding: ``quantize_e5m2`` works on the
float32 bit pattern with integer operations (fast enough for the 10^8-element
workloads); ``quantize_e5m2_f64`` spells the rounding out in float64
(frexp / ldexp / rint) and serves as a cross-check in tests. Both are pinned
against a brute-force nearest-value search.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E5M2_MAX_FINITE = 57344.0
# 0x7F = sign 0, exponent 31, mantissa 3: a NaN code. Used to poison bytes that
# must never reach the output (tail slots, unreferenced pages).
POISON_CODE = 0x7F

_F32_MAX_FINITE_E5M2 = np.float32(E5M2_MAX_FINITE).view(np.uint32)   # 0x47600000
_F32_MIN_NORMAL_E5M2 = np.float32(2.0 ** -14).view(np.uint32)        # 0x38800000


def quantize_e5m2(x) -> np.ndarray:
    """float32 array -> uint8 E5M2 codes, round-to-nearest-even, saturating."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if np.isnan(x32).any():
        raise ValueError("quantize_e5m2: NaN input")
    flat = x32.reshape(-1)
    if flat.size <= _CHUNK:
        return _quantize_block(flat).reshape(x32.shape)
    # numpy ufuncs release the GIL, so chunks quantise in parallel threads.
    out = np.empty(flat.size, dtype=np.uint8)
    starts = range(0, flat.size, _CHUNK)

    def work(s):
        out[s:s + _CHUNK] = _quantize_block(flat[s:s + _CHUNK])

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(work, starts))
    return out.reshape(x32.shape)


_CHUNK = 1 << 22


def _quantize_block(x32: np.ndarray) -> np.ndarray:
    u = x32.view(np.uint32)
    sign = (u >> np.uint32(31)).astype(np.uint8) << np.uint8(7)
    a = np.minimum(u & np.uint32(0x7FFFFFFF), _F32_MAX_FINITE_E5M2)

    # Normal E5M2 range: keep the float32 exponent and the top 2 mantissa bits,
    # rounding the 21 dropped bits to nearest even (a carry into the exponent is
    # the correct next binade). Re-bias 127 -> 15, i.e. subtract 112 << 2.
    lsb = (a >> np.uint32(21)) & np.uint32(1)
    r = (a + np.uint32(0xFFFFF) + lsb) >> np.uint32(21)
    normal_code = r.astype(np.int32) - (112 << 2)

    # Subnormal E5M2 range: the grid is m * 2^-16; |x| * 2^16 is exact in
    # float32 and rint rounds half to even. The result 4 is code 4 = 2^-14.
    mag = np.minimum(a, _F32_MIN_NORMAL_E5M2).view(np.float32)
    sub_code = np.rint(mag * np.float32(65536.0)).astype(np.int32)

    code = np.where(a >= _F32_MIN_NORMAL_E5M2, normal_code, sub_code)
    return code.astype(np.uint8) | sign


def quantize_e5m2_f64(x) -> np.ndarray:
    """The same rounding written out in float64 (slow; used to cross-check)."""
    x32 = np.asarray(x, dtype=np.float32)
    if np.isnan(x32).any():
        raise ValueError("quantize_e5m2_f64: NaN input")
    a = np.minimum(np.abs(x32.astype(np.float64)), E5M2_MAX_FINITE)
    neg = np.signbit(x32)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -14
    code[sub] = np.rint(a[sub] * 65536.0).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        av = a[nrm]
        _, ex = np.frexp(av)          # av = f * 2^ex, f in [0.5, 1)
        e = ex.astype(np.int64) - 1   # av = (2f) * 2^e, 2f in [1, 2)
        qq = np.rint(np.ldexp(av, (2 - e).astype(np.int32))).astype(np.int64)  # 4..8
        carry = qq == 8
        e = e + carry
        qq = np.where(carry, 4, qq)
        code[nrm] = ((e + 15) << 2) + (qq - 4)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


E4M3_MAX_FINITE = 448.0


def quantize_e4m3(x) -> np.ndarray:
    """float -> OCP E4M3 codes (uint8): round to nearest even, saturating at +-448.

    Input generation only (the kernels decode E4M3; they never encode it):
    values are clipped to the largest finite magnitude and converted by
    torch's float8_e4m3fn cast, which rounds to nearest even.
    """
    import torch
    a = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX_FINITE, E4M3_MAX_FINITE)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()
