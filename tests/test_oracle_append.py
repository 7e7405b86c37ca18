"""Pins for the oracle's KV append (E5M2 encoding + page scatter), CPU only.

The encoder is checked against a brute-force nearest search over every
finite code for all 65536 binary16 inputs, against hand-worked anchors and
against the round trip of every code; the scatter is checked through the
decode oracle's own gather (append then gather == old tokens + new token).
"""

import numpy as np
import pytest

import oracle
from oracle.e5m2 import E5M2_TABLE
from workloads import quantize_e5m2


def _finite_codes():
    codes = np.arange(256)
    e = (codes >> 2) & 31
    return codes[e != 31]


def test_encode_is_nearest_finite_value_for_every_fp16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float64)
    keep = ~np.isnan(x) & ~np.isinf(x)
    x = x[keep]
    got = oracle.encode_e5m2(x).astype(np.int64)
    fin = _finite_codes()
    # The sign is kept: candidates are the finite codes of the input's sign.
    sign = np.signbit(x)
    assert np.array_equal((got >> 7) == 1, sign)
    vals = E5M2_TABLE[fin]
    pos = fin[fin < 128]
    neg = fin[fin >= 128]
    for chunk in range(0, x.size, 8192):
        xs = x[chunk:chunk + 8192]
        gs = got[chunk:chunk + 8192]
        sg = sign[chunk:chunk + 8192]
        for cand, mask in ((pos, ~sg), (neg, sg)):
            if not mask.any():
                continue
            xv = xs[mask][:, None]
            d = np.abs(xv - E5M2_TABLE[cand][None, :])
            dmin = d.min(axis=1)
            dg = np.abs(xs[mask] - E5M2_TABLE[gs[mask]])
            assert np.array_equal(dg, dmin), "not the nearest finite value"
            ties = (d == dmin[:, None]).sum(axis=1) > 1
            # +-0 compete only with each other's sign twin, which is excluded.
            assert (gs[mask][ties] % 2 == 0).all(), "tie not resolved to the even code"
    del vals


def test_encode_roundtrips_every_finite_code():
    fin = _finite_codes()
    assert np.array_equal(oracle.encode_e5m2(E5M2_TABLE[fin]).astype(np.int64), fin)


def test_encode_midpoints_go_to_the_even_code():
    for base in (0, 128):
        for c in range(base, base + 0x7B):
            a, b = E5M2_TABLE[c], E5M2_TABLE[c + 1]
            mid = (a + b) / 2.0
            even = c if c % 2 == 0 else c + 1
            assert oracle.encode_e5m2(mid) == even
            assert oracle.encode_e5m2(np.nextafter(mid, a)) == c
            assert oracle.encode_e5m2(np.nextafter(mid, b)) == c + 1


@pytest.mark.parametrize("x,code", [
    (1.0, 0x3C), (1.25, 0x3D), (1.125, 0x3C), (1.375, 0x3E), (-1.5, 0xBE),
    (57344.0, 0x7B), (60000.0, 0x7B), (1e30, 0x7B), (np.inf, 0x7B), (-np.inf, 0xFB),
    (2.0 ** -16, 0x01), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02), (-2.0 ** -18, 0x80),
    (0.0, 0x00), (-0.0, 0x80), (np.nan, 0x7F), (-np.nan, 0xFF),
])
def test_encode_anchors(x, code):
    # Worked by hand from the format: 1.125 lies halfway between 1.0 (0x3C)
    # and 1.25 (0x3D) and goes to the even code; values past 57344 saturate.
    assert int(oracle.encode_e5m2(x)) == code


def test_encode_agrees_with_the_data_quantizer():
    # Two independently pinned implementations of the same reading.
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-14, 12, 200000))).astype(np.float32)
    assert np.array_equal(oracle.encode_e5m2(x), quantize_e5m2(x))


def _pools(rng, num_pages, hkv, P=16, D=128):
    k = rng.integers(0, 256, size=(num_pages, hkv, P, D), dtype=np.uint8)
    v = rng.integers(0, 256, size=(num_pages, hkv, P, D), dtype=np.uint8)
    return k, v


def test_append_then_gather_is_old_tokens_plus_new_token():
    rng = np.random.default_rng(11)
    hkv, P, max_pages = 2, 16, 4
    lens_after = np.array([1, 16, 17, 33, 64, 0, -3, 65, 40], dtype=np.int64)
    B = lens_after.size
    num_pages = B * max_pages
    k, v = _pools(rng, num_pages, hkv)
    bt = rng.permutation(num_pages).reshape(B, max_pages).astype(np.int32)
    k_new = rng.standard_normal((B, hkv, 128)).astype(np.float16)
    v_new = (rng.standard_normal((B, hkv, 128)) * 3).astype(np.float16)
    k2, v2 = oracle.append_kv(k, v, bt, lens_after, k_new, v_new)
    capacity = max_pages * P
    touched = np.zeros(k.shape, dtype=bool)
    for b in range(B):
        n = int(lens_after[b])
        if n <= 0 or n > capacity:
            continue
        for h in range(hkv):
            before_k = oracle.gather_tokens(k, bt, b, h, n - 1)
            after_k = oracle.gather_tokens(k2, bt, b, h, n)
            after_v = oracle.gather_tokens(v2, bt, b, h, n)
            assert np.array_equal(after_k[:n - 1], before_k, equal_nan=True)   # random codes hold NaNs
            assert np.array_equal(after_k[n - 1], E5M2_TABLE[oracle.encode_e5m2(k_new[b, h])])
            assert np.array_equal(after_v[n - 1], E5M2_TABLE[oracle.encode_e5m2(v_new[b, h])])
        t = n - 1
        touched[bt[b, t // P], :, t % P, :] = True
    # Nothing else changed: lengths <= 0 or past the capacity write nothing.
    assert np.array_equal(k2[~touched], k[~touched])
    assert np.array_equal(v2[~touched], v[~touched])
    assert touched.sum() == 6 * hkv * 128   # lengths 1, 16, 17, 33, 64, 40


def test_append_then_attend_equals_attention_with_the_new_token():
    # The appended token takes part in the next decode exactly like any
    # cached token: attention over the pools after the append equals the
    # plain definition over the old tokens plus the encoded new token.
    rng = np.random.default_rng(12)
    hkv, hq, P, max_pages = 2, 8, 16, 3
    lens_after = np.array([5, 16, 17, 48], dtype=np.int64)
    B = lens_after.size
    k, v = _pools(rng, B * max_pages, hkv)
    # Replace NaN/inf codes so the attention is finite.
    k[((k >> 2) & 31) == 31] = 0x3C
    v[((v >> 2) & 31) == 31] = 0x3C
    bt = rng.permutation(B * max_pages).reshape(B, max_pages).astype(np.int32)
    q = rng.standard_normal((B, hq, 128)).astype(np.float16)
    k_new = rng.standard_normal((B, hkv, 128)).astype(np.float16)
    v_new = rng.standard_normal((B, hkv, 128)).astype(np.float16)
    k2, v2 = oracle.append_kv(k, v, bt, lens_after, k_new, v_new)
    out = oracle.decode_attention(q, k2, v2, bt, lens_after, 0.0883883461356163)
    G = hq // hkv
    for b in range(B):
        n = int(lens_after[b])
        for hqi in range(hq):
            h = hqi // G
            K = np.vstack([oracle.gather_tokens(k, bt, b, h, n - 1),
                           E5M2_TABLE[oracle.encode_e5m2(k_new[b, h])][None, :]])
            V = np.vstack([oracle.gather_tokens(v, bt, b, h, n - 1),
                           E5M2_TABLE[oracle.encode_e5m2(v_new[b, h])][None, :]])
            z = np.float64(np.float32(0.0883883461356163)) * (K @ q[b, hqi].astype(np.float64))
            p = np.exp(z - z.max())
            ref = (p @ V) / p.sum()
            np.testing.assert_allclose(out[b, hqi], ref, rtol=1e-12, atol=1e-12)


def test_planted_append_mistakes_are_caught():
    # A slot off by one, or the pages of K and V exchanged, must fail the
    # gather check above: rerun its core with a mutated result.
    rng = np.random.default_rng(13)
    k, v = _pools(rng, 8, 1)
    bt = np.arange(8, dtype=np.int32).reshape(2, 4)
    lens = np.array([5, 20])
    k_new = rng.standard_normal((2, 1, 128)).astype(np.float16) * 7
    v_new = rng.standard_normal((2, 1, 128)).astype(np.float16) * 7
    k2, v2 = oracle.append_kv(k, v, bt, lens, k_new, v_new)

    def ok(kk, vv):
        for b in range(2):
            n = int(lens[b])
            if not np.array_equal(oracle.gather_tokens(kk, bt, b, 0, n)[n - 1],
                                  E5M2_TABLE[oracle.encode_e5m2(k_new[b, 0])]):
                return False
            if not np.array_equal(oracle.gather_tokens(vv, bt, b, 0, n)[n - 1],
                                  E5M2_TABLE[oracle.encode_e5m2(v_new[b, 0])]):
                return False
        return True

    assert ok(k2, v2)
    assert not ok(v2, k2)                      # K and V exchanged
    shifted = k.copy()                         # written one slot too far
    for b in range(2):
        t = int(lens[b])
        shifted[bt[b, t // 16], :, t % 16, :] = oracle.encode_e5m2(k_new[b])
    assert not ok(shifted, v2)
