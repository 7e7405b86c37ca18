"""Pins for the oracle's page-subset decode (attention over selected pages), CPU only."""

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


def _visible_pages_brute(sel_row, count, n, P, S):
    # A page entry counts when it is a page the sequence uses and is a strict
    # new maximum of the in-range entries before it (the kept entries are
    # exactly those records).
    used = (n + P - 1) // P
    count = min(max(count, 0), S)
    best = -1
    pages = set()
    for j in range(count):
        p = int(sel_row[j])
        if p < 0 or p >= used:
            continue
        if p > best:
            pages.add(p)
            best = p
    return pages


def _brute(q, k, v, bt, lens, sel, counts, scale, include_tail_slots=False):
    # Explicit loops, math.exp and math.fsum over every token of the
    # sequence, keeping those whose page is visible.
    B, Hq, D = q.shape
    Hkv, P = k.shape[1], k.shape[2]
    G = Hq // Hkv
    s = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = max(0, min(int(lens[b]), bt.shape[1] * P))
        pages = _visible_pages_brute(sel[b], int(counts[b]), n, P, sel.shape[1])
        limit = -(-n // P) * P if include_tail_slots else n
        ts = [t for t in range(limit) if t // P in pages]
        for hq in range(Hq):
            h = hq // G
            if not ts:
                continue
            z = []
            for t in ts:
                kt = E5M2_TABLE[k[bt[b, t // P], h, t % P]]
                z.append(s * math.fsum(float(q[b, hq, d]) * kt[d] for d in range(D)))
            zm = max(z)
            w = [math.exp(zz - zm) for zz in z]
            lsum = math.fsum(w)
            for d in range(D):
                out[b, hq, d] = math.fsum(
                    w[i] * E5M2_TABLE[v[bt[b, t // P], h, t % P, d]] for i, t in enumerate(ts)) / lsum
    return out


def test_pages_match_brute_force():
    rng = np.random.default_rng(71)
    k, v, bt = _small(rng, 4, 2, 4)
    lens = np.array([61, 33, 0, 16])
    S = 6
    sel = np.array([[0, 2, 3, 1, 9, 3],      # 1 after 3 skipped, 9 out of range, 3 repeated
                    [2, 0, 1, 2, -1, 0],     # 0 and 1 after 2 skipped
                    [0, 1, 2, 3, 4, 5],      # empty sequence
                    [-3, 0, 0, 0, 0, 0]],    # negative entry skipped, then page 0
                   dtype=np.int32)
    counts = np.array([6, 5, 6, 2])
    q = rng.standard_normal((4, 4, 8)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.3)
    ref = _brute(q, k, v, bt, lens, sel, counts, 0.3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert (got[2] == 0).all()
    assert oracle.kept_pages(sel, counts, 61, 16, 0) == [0, 2, 3]
    assert oracle.kept_pages(sel, counts, 33, 16, 1) == [2]
    assert oracle.kept_pages(sel, counts, 16, 16, 3) == [0]


def test_planted_mistakes_are_caught_by_the_brute_force():
    # Mistakes an implementation could make, planted in the brute force:
    # attending the slots past n of the last page, and an off-by-one in the
    # page of a token. Each must change the result.
    rng = np.random.default_rng(72)
    k, v, bt = _small(rng, 2, 1, 3)
    lens = np.array([37, 40])
    sel = np.array([[0, 2], [1, 2]], dtype=np.int32)
    counts = np.array([2, 2])
    q = rng.standard_normal((2, 4, 8)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.5)
    wrong_tail = _brute(q, k, v, bt, lens, sel, counts, 0.5, include_tail_slots=True)
    assert np.abs(got - wrong_tail).max() > 1e-6
    shifted = sel + 1
    wrong_page = _brute(q, k, v, bt, lens, shifted, counts, 0.5)
    assert np.abs(got - wrong_page).max() > 1e-6


def test_every_page_in_order_is_plain_decode():
    rng = np.random.default_rng(73)
    k, v, bt = _small(rng, 5, 2, 4, D=128)
    lens = np.array([1, 17, 64, 0, 50])
    S = 4
    sel = np.tile(np.arange(S, dtype=np.int32), (5, 1))
    counts = np.full(5, S)
    q = rng.standard_normal((5, 16, 128)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.0883883461356163)
    ref = oracle.decode_attention(q, k, v, bt, lens, 0.0883883461356163)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_subset_is_plain_decode_over_the_kept_pages():
    # The kept pages, gathered into a block table of their own, with length
    # 16 * (pages - 1) plus what the last one holds: plain decode over that
    # table gives the same rows.
    rng = np.random.default_rng(74)
    P = 16
    k, v, bt = _small(rng, 3, 2, 6, D=128)
    lens = np.array([90, 96, 7])
    sel = np.array([[1, 3, 5, 0], [0, 5, 5, 2], [0, 0, 0, 0]], dtype=np.int32)
    counts = np.array([3, 4, 1])
    q = rng.standard_normal((3, 8, 128)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.1)
    bt2 = np.zeros_like(bt)
    lens2 = np.zeros(3, dtype=np.int64)
    for b in range(3):
        kept = oracle.kept_pages(sel, counts, int(lens[b]), P, b)
        for j, p in enumerate(kept):
            bt2[b, j] = bt[b, p]
        last = kept[-1]
        lens2[b] = P * (len(kept) - 1) + min(P, int(lens[b]) - P * last)
    assert list(lens2) == [16 + 16 + 10, 16 + 16, 7]
    ref = oracle.decode_attention(q, k, v, bt2, lens2, 0.1)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_single_page_single_token_and_empty_selection():
    rng = np.random.default_rng(75)
    k, v, bt = _small(rng, 3, 1, 3, D=128)
    lens = np.array([33, 40, 40])
    # Sequence 0 keeps only page 2, which holds token 32 alone: the row is
    # that token's V exactly. Sequence 1 selects nothing; sequence 2 only
    # out-of-range pages. Both give zero rows.
    sel = np.array([[2, 0], [0, 1], [3, 7]], dtype=np.int32)
    counts = np.array([1, 0, 2])
    q = rng.standard_normal((3, 4, 128)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.2)
    v_row = E5M2_TABLE[v[bt[0, 2], 0, 0]]
    for hq in range(4):
        assert np.array_equal(got[0, hq], v_row)
    assert (got[1] == 0).all() and (got[2] == 0).all()


def test_unselected_pages_and_tail_slots_never_matter():
    rng = np.random.default_rng(76)
    k, v, bt = _small(rng, 2, 2, 4, D=128)
    lens = np.array([50, 64])
    sel = np.array([[1, 3], [0, 2]], dtype=np.int32)
    counts = np.array([2, 2])
    q = rng.standard_normal((2, 16, 128)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.3)
    k2, v2 = k.copy(), v.copy()
    for b, p in [(0, 0), (0, 2), (1, 1), (1, 3)]:      # unselected pages: NaN codes
        k2[bt[b, p]] = 0x7F
        v2[bt[b, p]] = 0x7F
    k2[bt[0, 3], :, 2:] = 0x7F                          # slots past n = 50 in page 3
    v2[bt[0, 3], :, 2:] = 0x7F
    again = oracle.decode_attention_pages(q, k2, v2, bt, lens, sel, counts, 0.3)
    assert np.array_equal(got, again)


def test_physical_page_permutation_does_not_matter():
    rng = np.random.default_rng(77)
    k, v, bt = _small(rng, 2, 2, 4, D=128)
    lens = np.array([55, 49])
    sel = np.array([[0, 1, 3, 3], [2, 3, 0, 0]], dtype=np.int32)
    counts = np.array([4, 2])
    q = rng.standard_normal((2, 8, 128)).astype(np.float16)
    got = oracle.decode_attention_pages(q, k, v, bt, lens, sel, counts, 0.25)
    perm = rng.permutation(k.shape[0])
    inv = np.argsort(perm)
    kp, vp = k[perm], v[perm]                         # page i moves to slot inv[i]
    again = oracle.decode_attention_pages(q, kp, vp, inv[bt].astype(np.int32), lens, sel, counts, 0.25)
    np.testing.assert_allclose(got, again, rtol=0, atol=0)
