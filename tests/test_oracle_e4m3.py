"""Pins for the oracle's E4M3 decode and the FP8 attention with per-tensor scales (CPU)."""

import numpy as np
import pytest
import torch

import oracle
from oracle.e4m3 import E4M3_TABLE
from oracle.e5m2 import E5M2_TABLE


def test_every_e4m3_code_matches_torch_float8_e4m3fn():
    # An independent implementation of the same OCP format: torch's CPU
    # float8_e4m3fn conversion.
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_every_e5m2_code_matches_torch_float8_e5m2():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(E5M2_TABLE), nan)
    assert np.array_equal(E5M2_TABLE[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x39, 1.125), (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x00, 0.0), (0x80, -0.0), (0x40, 2.0),
    (0x77, 240.0), (0x7F, np.nan), (0xFF, np.nan), (0x78, 256.0),
])
def test_e4m3_anchors(code, value):
    # Worked by hand: 0x38 = exponent 7 (bias 7), mantissa 0; 0x7E = 1.75 * 2^8;
    # 0x78 = 2^8 (exponent 15 is finite in E4M3 except with mantissa 7).
    got = oracle.decode_e4m3(code)
    if np.isnan(value):
        assert np.isnan(got)
    else:
        assert got == value and np.signbit(got) == np.signbit(value)


def _pools(rng, num_pages, hkv, table_ok):
    shape = (num_pages, hkv, 16, 128)
    k = rng.choice(table_ok, size=shape).astype(np.uint8)
    v = rng.choice(table_ok, size=shape).astype(np.uint8)
    return k, v


def test_fp8_attention_reduces_to_the_e5m2_oracles():
    rng = np.random.default_rng(41)
    finite = np.array([c for c in range(256) if np.isfinite(E5M2_TABLE[c]) and abs(E5M2_TABLE[c]) < 64])
    k, v = _pools(rng, 12, 2, finite)
    bt = rng.permutation(12).reshape(3, 4).astype(np.int32)
    lens = np.array([20, 64, 3])
    q1 = rng.standard_normal((3, 16, 128)).astype(np.float16)
    a = oracle.decode_attention_fp8(q1, k, v, bt, lens, 0.09)
    assert np.array_equal(a, oracle.decode_attention(q1, k, v, bt, lens, 0.09))
    q3 = rng.standard_normal((3, 2, 16, 128)).astype(np.float16)
    b = oracle.decode_attention_fp8(q3, k, v, bt, lens, 0.09)
    assert np.array_equal(b, oracle.decode_attention_multi(q3, k, v, bt, lens, 0.09))


def test_e4m3_equals_e5m2_on_values_both_formats_hold():
    # Values (1 + m/4) 2^e with e in [-6, 8] exist in both formats; a cache of
    # such values gives the same attention whichever format encodes it.
    common = [c for c in range(256)
              if np.isfinite(E5M2_TABLE[c]) and E5M2_TABLE[c] != 0
              and 2.0 ** -6 <= abs(E5M2_TABLE[c]) <= 256]
    e4_of = {}
    for c in common:
        match = np.nonzero(E4M3_TABLE == E5M2_TABLE[c])[0]
        assert match.size == 1
        e4_of[c] = int(match[0])
    rng = np.random.default_rng(42)
    k5, v5 = _pools(rng, 8, 1, np.array(common))
    lut = np.zeros(256, dtype=np.uint8)
    for c, d in e4_of.items():
        lut[c] = d
    k4, v4 = lut[k5], lut[v5]
    bt = rng.permutation(8).reshape(2, 4).astype(np.int32)
    lens = np.array([50, 9])
    q = rng.standard_normal((2, 4, 128)).astype(np.float16)
    a = oracle.decode_attention_fp8(q, k5, v5, bt, lens, 0.01, kv_format="e5m2")
    b = oracle.decode_attention_fp8(q, k4, v4, bt, lens, 0.01, kv_format="e4m3")
    assert np.array_equal(a, b)


def test_scales_act_as_stated():
    # v_scale multiplies the output; k_scale multiplies the softmax scale
    # (powers of two keep both identities exact).
    rng = np.random.default_rng(43)
    finite = np.array([c for c in range(256) if np.isfinite(E4M3_TABLE[c])])
    k, v = _pools(rng, 6, 2, finite)
    bt = rng.permutation(6).reshape(2, 3).astype(np.int32)
    lens = np.array([40, 17])
    q = rng.standard_normal((2, 8, 128)).astype(np.float16)
    base = oracle.decode_attention_fp8(q, k, v, bt, lens, 0.02, kv_format="e4m3")
    vs = oracle.decode_attention_fp8(q, k, v, bt, lens, 0.02, kv_format="e4m3", v_scale=0.125)
    assert np.array_equal(vs, base * 0.125)
    ks = oracle.decode_attention_fp8(q, k, v, bt, lens, 0.02, kv_format="e4m3", k_scale=4.0)
    sc = oracle.decode_attention_fp8(q, k, v, bt, lens, 0.08, kv_format="e4m3")
    np.testing.assert_allclose(ks, sc, rtol=1e-13, atol=1e-300)
    assert not np.allclose(ks, base)
