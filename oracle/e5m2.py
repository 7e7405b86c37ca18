"""Closed-form decode of FP8 E5M2 codes (test infrastructure only).

The pages ("[Kernel][SM70] Pipeline batched E5M2 XQA decode", section Purpose
and the deployment line listing an FP8 E5M2 KV cache) name the format but do
not spell it out. Reading taken: the OCP 8-bit floating-point E5M2 encoding,
which is one sign bit, a 5-bit exponent with bias 15 and a 2-bit mantissa,
with IEEE-style subnormals, infinities and NaNs:

    s = bit 7, e = bits 6..2, m = bits 1..0
    e == 0        value = (-1)^s * m * 2^-16           (subnormal, m = 0 is +-0)
    1 <= e <= 30  value = (-1)^s * (4 + m) * 2^(e - 17)  (= 2^(e-15) * (1 + m/4))
    e == 31       m == 0 -> (-1)^s * inf, otherwise NaN

The largest finite magnitude is code 0x7B = 1.75 * 2^15 = 57344.
"""

import numpy as np

E5M2_MAX_FINITE = 57344.0


def decode_e5m2(codes) -> np.ndarray:
    """Decode an array of E5M2 codes (any integer dtype, values 0..255) to float64."""
    b = np.asarray(codes).astype(np.int64)
    if b.size and (b.min() < 0 or b.max() > 255):
        raise ValueError("E5M2 codes must lie in 0..255")
    s = b >> 7
    e = (b >> 2) & 31
    m = b & 3
    sign = np.where(s == 1, -1.0, 1.0)
    out = np.empty(b.shape, dtype=np.float64)

    sub = e == 0
    out[sub] = sign[sub] * m[sub].astype(np.float64) * 2.0 ** -16

    nrm = (e >= 1) & (e <= 30)
    out[nrm] = sign[nrm] * np.ldexp((4 + m[nrm]).astype(np.float64), e[nrm] - 17)

    inf = (e == 31) & (m == 0)
    out[inf] = sign[inf] * np.inf

    nan = (e == 31) & (m != 0)
    out[nan] = np.nan
    return out


# The definition above applied once to every code; large inputs are decoded by
# indexing this table, which is the same function evaluated in advance.
E5M2_TABLE = decode_e5m2(np.arange(256))
E5M2_TABLE.setflags(write=False)
