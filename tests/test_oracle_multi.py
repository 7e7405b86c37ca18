"""Pins for the oracle's multi-token (causal) decode, CPU only."""

import math

import numpy as np

import oracle
from oracle.e5m2 import E5M2_TABLE


def _small(rng, B, hkv, pages_per_seq, D=8, P=16):
    num_pages = B * pages_per_seq + 1
    k = rng.integers(0, 256, size=(num_pages, hkv, P, D), dtype=np.uint8)
    v = rng.integers(0, 256, size=(num_pages, hkv, P, D), dtype=np.uint8)
    # Keep codes finite: exponent field 31 is inf/NaN.
    k[((k >> 2) & 31) >= 24] &= 0x83
    v[((v >> 2) & 31) >= 24] &= 0x83
    bt = rng.permutation(num_pages)[:B * pages_per_seq].reshape(B, pages_per_seq).astype(np.int32)
    return k, v, bt


def _brute(q, k, v, bt, lens, scale):
    # Explicit loops, math.exp and math.fsum: token t is visible to query
    # token j when t <= n - M + j.
    B, M, Hq, D = q.shape
    Hkv, P = k.shape[1], k.shape[2]
    G = Hq // Hkv
    s = float(np.float32(scale))
    out = np.zeros((B, M, Hq, D))
    for b in range(B):
        n = max(0, min(int(lens[b]), bt.shape[1] * P))
        for j in range(M):
            for hq in range(Hq):
                h = hq // G
                ts = [t for t in range(n) if t <= n - M + j]
                if not ts:
                    continue
                z = []
                for t in ts:
                    kt = E5M2_TABLE[k[bt[b, t // P], h, t % P]]
                    z.append(s * math.fsum(float(q[b, j, hq, d]) * kt[d] for d in range(D)))
                zm = max(z)
                w = [math.exp(zz - zm) for zz in z]
                lsum = math.fsum(w)
                for d in range(D):
                    out[b, j, hq, d] = math.fsum(
                        w[i] * E5M2_TABLE[v[bt[b, t // P], h, t % P, d]] for i, t in enumerate(ts)) / lsum
    return out


def test_multi_matches_brute_force_with_causal_loops():
    rng = np.random.default_rng(31)
    k, v, bt = _small(rng, 3, 2, 2)
    lens = np.array([19, 2, 0])          # n < M gives zero rows for the early queries
    q = rng.standard_normal((3, 3, 4, 8)).astype(np.float16)
    got = oracle.decode_attention_multi(q, k, v, bt, lens, 0.3)
    ref = _brute(q, k, v, bt, lens, 0.3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert (got[1, 0] == 0).all() and (got[2] == 0).all()
    assert (got[1, 1] != 0).any()


def test_one_query_token_is_the_single_token_decode():
    rng = np.random.default_rng(32)
    k, v, bt = _small(rng, 4, 2, 3, D=128)
    lens = np.array([1, 17, 48, 0])
    q = rng.standard_normal((4, 1, 8, 128)).astype(np.float16)
    got = oracle.decode_attention_multi(q, k, v, bt, lens, 0.0883883461356163)
    ref = oracle.decode_attention(q[:, 0], k, v, bt, lens, 0.0883883461356163)
    assert np.array_equal(got[:, 0], ref)


def test_query_j_sees_the_prefix_ending_at_its_position():
    # Each query row equals a single-token decode over the lengths n - M + j + 1.
    rng = np.random.default_rng(33)
    k, v, bt = _small(rng, 3, 1, 3, D=128)
    lens = np.array([40, 5, 33])
    M = 4
    q = rng.standard_normal((3, M, 4, 128)).astype(np.float16)
    got = oracle.decode_attention_multi(q, k, v, bt, lens, 0.1)
    for j in range(M):
        single = oracle.decode_attention(q[:, j], k, v, bt, lens - M + j + 1, 0.1)
        np.testing.assert_allclose(got[:, j], single, rtol=1e-13, atol=0)


def test_last_token_changes_only_the_last_query():
    rng = np.random.default_rng(34)
    k, v, bt = _small(rng, 1, 1, 2, D=128)
    lens = np.array([27])
    q = rng.standard_normal((1, 3, 2, 128)).astype(np.float16)
    # A tiny scale keeps the weights near uniform, so every visible token's V
    # shows in the output.
    a = oracle.decode_attention_multi(q, k, v, bt, lens, 1e-6)
    t = 26
    k2, v2 = k.copy(), v.copy()
    k2[bt[0, t // 16], 0, t % 16, :] ^= 0x04     # change the last token's K and V
    v2[bt[0, t // 16], 0, t % 16, :] ^= 0x04
    b = oracle.decode_attention_multi(q, k2, v2, bt, lens, 1e-6)
    assert np.array_equal(a[0, :2], b[0, :2])
    assert not np.array_equal(a[0, 2], b[0, 2])


def test_planted_causal_mistakes_are_caught():
    rng = np.random.default_rng(35)
    k, v, bt = _small(rng, 2, 1, 2)
    lens = np.array([20, 9])
    q = rng.standard_normal((2, 3, 2, 8)).astype(np.float16)
    ref = _brute(q, k, v, bt, lens, 0.5)
    # (1) the limit off by one: query j sees one token fewer.
    off = np.zeros_like(ref)
    for j in range(3):
        off[:, j] = oracle.decode_attention(q[:, j], k, v, bt, lens - 3 + j, 0.5)
    assert not np.allclose(off, ref, rtol=1e-6, atol=1e-9)
    # (2) query tokens read head-major instead of token-major.
    swapped = np.ascontiguousarray(q.transpose(0, 2, 1, 3)).reshape(q.shape)
    assert not np.allclose(oracle.decode_attention_multi(swapped, k, v, bt, lens, 0.5), ref,
                           rtol=1e-6, atol=1e-9)
