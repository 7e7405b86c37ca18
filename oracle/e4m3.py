"""Closed-form decode of FP8 E4M3 codes (test infrastructure only).

The page "[Kernel][WIP] Follow up FlashNext batch HC fusion and QSA route
audit" (section Test Result) names E4M3 as a cache format still awaiting
quality admission, without spelling the format out. Reading taken: the
OCP 8-bit floating-point E4M3 encoding ("E4M3FN"): one sign bit, a 4-bit
exponent with bias 7 and a 3-bit mantissa, subnormals, no infinities, and
NaN only for exponent 15 with mantissa 7:

    s = bit 7, e = bits 6..3, m = bits 2..0
    e == 0                 value = (-1)^s * m * 2^-9             (subnormal, m = 0 is +-0)
    1 <= e, not (15, 7)    value = (-1)^s * (8 + m) * 2^(e - 10)  (= 2^(e-7) * (1 + m/8))
    e == 15 and m == 7     NaN

The largest finite magnitude is code 0x7E = 1.75 * 2^8 = 448.
"""

import numpy as np

E4M3_MAX_FINITE = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """Decode an array of E4M3 codes (any integer dtype, values 0..255) to float64."""
    b = np.asarray(codes).astype(np.int64)
    if b.size and (b.min() < 0 or b.max() > 255):
        raise ValueError("E4M3 codes must lie in 0..255")
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    sign = np.where(s == 1, -1.0, 1.0)
    out = np.empty(b.shape, dtype=np.float64)
    sub = e == 0
    out[sub] = sign[sub] * m[sub].astype(np.float64) * 2.0 ** -9
    nrm = ~sub
    out[nrm] = sign[nrm] * np.ldexp((8 + m[nrm]).astype(np.float64), e[nrm] - 10)
    nan = (e == 15) & (m == 7)
    out[nan] = np.nan
    return out


# The definition above evaluated once for every code.
E4M3_TABLE = decode_e4m3(np.arange(256))
E4M3_TABLE.setflags(write=False)
