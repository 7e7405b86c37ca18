"""Pins for the oracle's E5M2 decode (CPU only).

The closed form in oracle/e5m2.py is checked against two things it does not
use: the IEEE binary16 value of the code placed in the high byte of a 16-bit
word (E5M2 shares binary16's sign, exponent width and bias, so the byte is
exactly the top half of a binary16 number), and hand-worked anchors.
"""

import math
import os

import numpy as np

from oracle import decode_e5m2, E5M2_TABLE, E5M2_MAX_FINITE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e5m2_anchors.txt")


def _fp16_view(codes):
    words = (np.asarray(codes, dtype=np.uint16) << 8).astype(np.uint16)
    return words.view(np.float16).astype(np.float64)


def test_all_256_codes_match_binary16_high_byte():
    codes = np.arange(256)
    got = decode_e5m2(codes)
    ref = _fp16_view(codes)
    nan_ref = np.isnan(ref)
    assert (np.isnan(got) == nan_ref).all()
    fin = ~nan_ref
    assert (got[fin] == ref[fin]).all()
    assert (np.signbit(got[fin]) == np.signbit(ref[fin])).all()   # -0 kept


def test_code_classes():
    v = E5M2_TABLE
    assert np.isfinite(v).sum() == 248
    assert np.isinf(v).sum() == 2
    assert np.isnan(v).sum() == 6
    assert v[0x7B] == E5M2_MAX_FINITE == 57344.0
    assert np.nanmax(np.where(np.isfinite(v), v, np.nan)) == 57344.0


def test_hand_worked_anchors():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code_s, val_s = line.split()
            code, val = int(code_s, 16), float(val_s)
            got = float(decode_e5m2([code])[0])
            if math.isnan(val):
                assert math.isnan(got), hex(code)
            else:
                assert got == val, hex(code)
                assert math.copysign(1.0, got) == math.copysign(1.0, val), hex(code)
            n += 1
    assert n >= 20


def test_positive_finite_codes_are_value_ordered():
    # Codes 0x00..0x7B increase strictly in value; the quantizer's "even code"
    # tie rule relies on it.
    v = E5M2_TABLE[:0x7C]
    assert (np.diff(v) > 0).all()
    assert (E5M2_TABLE[0x80:0xFC] == -v).all()
