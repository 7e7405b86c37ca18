"""Pins for the generator's float32 -> E5M2 rounding (CPU only).

Reference: brute-force nearest value over all 124 non-negative finite codes,
ties to the even code, values taken from the binary16 high-byte view of each
code (independent of both quantizer implementations).
"""

import numpy as np
import pytest

from workloads.quantize import quantize_e5m2, quantize_e5m2_f64, E5M2_MAX_FINITE

POS_CODES = np.arange(0x7C)
POS_VALUES = (POS_CODES.astype(np.uint16) << 8).view(np.float16).astype(np.float64)


def brute_force(x32):
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    for i, xv in enumerate(x.reshape(-1)):
        a = min(abs(xv), E5M2_MAX_FINITE)
        d = np.abs(POS_VALUES - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 2:
            c = best[0] if best[0] % 2 == 0 else best[1]
        else:
            c = best[0]
        if np.signbit(xv):
            c |= 0x80
        out.reshape(-1)[i] = c
    return out


def _critical_points():
    pts = []
    for i in range(len(POS_VALUES) - 1):
        mid = np.float32((POS_VALUES[i] + POS_VALUES[i + 1]) / 2)   # exact in float32
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))]
        pts += [np.float32(POS_VALUES[i])]
    pts += [np.float32(57344.0), np.float32(61440.0), np.float32(1e6),
            np.finfo(np.float32).max, np.float32(2.0 ** -17), np.float32(2.0 ** -18),
            np.float32(1e-30), np.float32(0.0)]
    pts = np.array(pts, dtype=np.float32)
    return np.concatenate([pts, -pts])


@pytest.mark.parametrize("q", [quantize_e5m2, quantize_e5m2_f64])
def test_midpoints_and_neighbours_brute_force(q):
    x = _critical_points()
    assert (q(x) == brute_force(x)).all()


@pytest.mark.parametrize("q", [quantize_e5m2, quantize_e5m2_f64])
def test_random_values_brute_force(q):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-5).astype(np.float32),
        (rng.standard_normal(1000) * 3e4).astype(np.float32),
    ])
    assert (q(x) == brute_force(x)).all()


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c >> 2) & 31 != 31], dtype=np.uint16)
    vals = (codes << 8).view(np.float16).astype(np.float32)
    assert (quantize_e5m2(vals) == codes.astype(np.uint8)).all()


def test_saturation_and_specials():
    x = np.array([57344.0, 61440.0, 1e6, np.inf, -np.inf, -61440.0,
                  np.finfo(np.float32).max], dtype=np.float32)
    assert quantize_e5m2(x).tolist() == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB, 0x7B]
    assert quantize_e5m2(np.array([-1e-30, -0.0], dtype=np.float32)).tolist() == [0x80, 0x80]
    with pytest.raises(ValueError):
        quantize_e5m2(np.array([np.nan], dtype=np.float32))


def test_no_double_rounding_through_float16():
    # 1.375 - 2^-20 is just below the 1.25 / 1.5 midpoint: the direct rounding
    # gives 1.25 (0x3D). Rounding to float16 first lands exactly on the
    # midpoint, which then ties to the even code 1.5 (0x3E).
    x = np.array([1.375 - 2.0 ** -20], dtype=np.float32)
    assert quantize_e5m2(x)[0] == 0x3D
    via16 = x.astype(np.float16).astype(np.float32)
    assert quantize_e5m2(via16)[0] == 0x3E


def test_fast_and_f64_agree_large_parallel_path():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1 << 23, dtype=np.float32)
    x[: 1 << 20] *= np.float32(1e-4)
    x[1 << 20: 1 << 21] *= np.float32(2e4)
    assert (quantize_e5m2(x) == quantize_e5m2_f64(x)).all()


def test_e4m3_input_quantizer_is_nearest_even_saturating():
    # The E4M3 input generator against a brute-force nearest search over every
    # finite E4M3 value (ties to the even code, saturation at +-448).
    from oracle.e4m3 import E4M3_TABLE
    from workloads.quantize import quantize_e4m3
    rng = np.random.default_rng(17)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-12, 7, 20000)),
        [0.0, -0.0, 448.0, 464.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875],
    ]).astype(np.float32)
    got = quantize_e4m3(x).astype(np.int64)
    fin = np.array([c for c in range(256) if np.isfinite(E4M3_TABLE[c])])
    for xi, gi in zip(x.astype(np.float64), got):
        same_sign = fin[(fin >= 128) == bool(np.signbit(xi))]
        d = np.abs(E4M3_TABLE[same_sign] - xi)
        best = same_sign[d == d.min()]
        assert gi in best, (xi, gi, best)
        if best.size > 1:
            assert gi % 2 == 0, (xi, gi, best)
