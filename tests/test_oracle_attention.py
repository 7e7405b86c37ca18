"""Pins for the float64 attention oracle (CPU only).

Each check comes from outside the oracle's own code: closed-form special
cases of softmax attention, invariances of the definition, a pure-Python
brute force written with math.exp / math.fsum over explicit loops, and the
exact log-sum-exp merge of split contexts. A last group plants plausible
mistakes into a copy of the oracle and checks that the pins catch them.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import attention as A
from workloads import make_custom, POISON_CODE
from workloads.quantize import quantize_e5m2


def _dec_bytes(code):
    """E5M2 value via the binary16 high-byte view (independent of the oracle)."""
    return float(np.array([code << 8], dtype=np.uint16).view(np.float16)[0])


def brute_force(w, b, hq):
    """out[b, hq, :] with explicit Python loops and math.exp / math.fsum."""
    G = w.num_q_heads // w.num_kv_heads
    h = hq // G
    n = int(w.context_lens[b])
    n = max(0, min(n, w.max_pages_per_seq * w.page_size))
    D = w.head_dim
    if n == 0:
        return [0.0] * D
    kp, vp = w.pools()
    s = float(np.float32(w.scale))
    qv = [float(x) for x in w.q[b, hq, :]]
    z = []
    for t in range(n):
        page = int(w.block_table[b][t // w.page_size])
        slot = t % w.page_size
        kt = [_dec_bytes(int(c)) for c in kp[page, h, slot, :]]
        z.append(s * math.fsum(qv[d] * kt[d] for d in range(D)))
    m = max(z)
    e = [math.exp(zt - m) for zt in z]
    den = math.fsum(e)
    out = []
    for d in range(D):
        num = math.fsum(e[t] * _dec_bytes(int(vp[int(w.block_table[b][t // w.page_size]), h, t % w.page_size, d]))
                        for t in range(n))
        out.append(num / den)
    return out


def run_oracle(w, **over):
    kp, vp = w.pools()
    args = dict(q=w.q, k_pages=kp, v_pages=vp, block_table=w.block_table,
                context_lens=w.context_lens, scale=w.scale)
    args.update(over)
    return oracle.decode_attention(**args)


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("ctx,hkv,hq,seed", [
    ([1, 17], 1, 8, 1),
    ([40, 5], 2, 16, 2),
    ([33], 2, 8, 3),
    ([0, 16, 31], 1, 8, 4),
])
def test_brute_force_tiny(ctx, hkv, hq, seed):
    w = make_custom(ctx, hkv, hq, seed, pool_pages=sum((c + 15) // 16 for c in ctx) + 3)
    out = run_oracle(w)
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            ref = np.array(brute_force(w, b, h))
            # Summation error is bounded relative to the row's largest |value|
            # (cancellation can leave single elements near zero).
            scale = max(np.abs(ref).max(), 1e-300)
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-12, atol=1e-12 * scale)


# ------------------------------------------------------------ special cases

def test_single_token_returns_its_v_row_exactly():
    w = make_custom([1, 1, 1], 2, 16, 10)
    out = run_oracle(w)
    for b in range(3):
        for hq in range(16):
            h = hq // 8
            v = oracle.decode_e5m2(w.v_tokens[b][0, h, :])
            assert (out[b, hq] == v).all()


def test_constant_v_returns_that_v():
    w = make_custom([70, 300], 2, 16, 11)
    for b in range(w.batch):
        w.v_tokens[b][:] = quantize_e5m2(np.float32([-2.5]))[0]
    out = run_oracle(w)
    np.testing.assert_allclose(out, -2.5, rtol=1e-14)


def test_uniform_k_gives_mean_of_v():
    w = make_custom([50, 129], 1, 8, 12)
    for b in range(w.batch):
        w.k_tokens[b][:] = w.k_tokens[b][0:1]
    out = run_oracle(w)
    for b in range(w.batch):
        mean = oracle.decode_e5m2(w.v_tokens[b][:, 0, :]).mean(axis=0)
        np.testing.assert_allclose(out[b], np.broadcast_to(mean, (8, 128)), rtol=1e-12, atol=1e-14)


def test_zero_scale_gives_mean_of_v():
    w = make_custom([45, 200], 2, 16, 13)
    out = run_oracle(w, scale=0.0)
    for b in range(w.batch):
        for hq in range(16):
            mean = oracle.decode_e5m2(w.v_tokens[b][:, hq // 8, :]).mean(axis=0)
            np.testing.assert_allclose(out[b, hq], mean, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("code", [0x3C, 0x5A, 0x7B, 0xFB])
def test_constant_column_shift_invariance(code):
    # Setting K[:, d0] to the same value for every token adds the same amount
    # to every score of a row; softmax is unchanged.
    w = make_custom([90, 37], 1, 8, 14)
    base = run_oracle(w)
    d0 = 77
    for b in range(w.batch):
        w.k_tokens[b][:, :, d0] = 0
    zero = run_oracle(w)
    for b in range(w.batch):
        w.k_tokens[b][:, :, d0] = code
    shifted = run_oracle(w)
    np.testing.assert_allclose(shifted, zero, rtol=1e-9, atol=1e-12)
    assert not np.allclose(base, zero, rtol=1e-9)   # the column does matter when not constant


def test_duplicated_query_rows_duplicate_outputs():
    w = make_custom([64, 100], 2, 16, 15)
    w.q[:, 3, :] = w.q[:, 5, :]
    out = run_oracle(w)
    assert (out[:, 3] == out[:, 5]).all()


def test_page_permutation_invariance():
    w = make_custom([100, 33, 250], 2, 16, 16, pool_pages=64)
    out = run_oracle(w)
    # Move every referenced page to a new random physical slot.
    kp, vp = w.pools()
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_pages)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    bt2 = perm[w.block_table].astype(np.int32)
    out2 = oracle.decode_attention(w.q, kp2, vp2, bt2, w.context_lens, w.scale)
    assert (out == out2).all()


def test_zero_and_negative_lengths_give_zero_rows():
    w = make_custom([0, 20], 1, 8, 17)
    ctx = w.context_lens.copy()
    ctx[0] = -5
    out = run_oracle(w, context_lens=ctx)
    assert (out[0] == 0).all()
    assert np.isfinite(out[1]).all() and (out[1] != 0).any()


def test_poison_never_reaches_output():
    # Tail slots, unreferenced pages and unused block-table entries hold the
    # NaN code; a finite output shows none of them was read.
    w = make_custom([1, 15, 17, 31], 2, 16, 18, pool_pages=40, max_pages_per_seq=4)
    kp, _ = w.pools()
    assert (kp[w.poison_page] == POISON_CODE).all()
    out = run_oracle(w)
    assert np.isfinite(out).all()


def test_length_clamped_to_block_table_capacity():
    w = make_custom([64], 1, 8, 19, max_pages_per_seq=4)
    out = run_oracle(w)
    ctx = w.context_lens.copy()
    ctx[0] = 10_000
    out_big = run_oracle(w, context_lens=ctx)
    assert (out == out_big).all()


# ------------------------------------------------- split contexts and merge

@pytest.mark.parametrize("n,seed", [(1, 1), (37, 2), (300, 3), (1025, 4)])
def test_merge_of_any_partition_equals_single_pass(n, seed):
    w = make_custom([n], 1, 8, 20 + seed)
    kp, vp = w.pools()
    K = A.gather_tokens(kp, w.block_table, 0, 0, n)
    V = A.gather_tokens(vp, w.block_table, 0, 0, n)
    rng = np.random.default_rng(seed)
    for hq in (0, 7):
        ref = oracle.decode_attention_row(w.q, kp, vp, w.block_table, w.context_lens, w.scale, 0, hq)
        for _ in range(4):
            cuts = np.sort(rng.choice(np.arange(0, n + 1), size=min(5, n + 1), replace=True))
            bounds = [0] + cuts.tolist() + [n]
            states = [oracle.partial_state(w.q[0, hq], K[a:b], V[a:b], w.scale)
                      for a, b in zip(bounds[:-1], bounds[1:])]
            got = oracle.merge_states(states)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_merge_handles_empty_parts_and_large_offsets():
    # States with very different maxima (range stress) merge exactly.
    D = 4
    s1 = (0.0, 2.0, np.array([1.0, 2.0, 3.0, 4.0]))
    s2 = (-800.0, 5.0, np.array([9.0, 9.0, 9.0, 9.0]))
    empty = (-np.inf, 0.0, np.zeros(D))
    got = oracle.merge_states([empty, s1, s2, empty])
    np.testing.assert_allclose(got, s1[2] / s1[1], rtol=1e-15)


# -------------------------------------------------- planted mistakes caught

def _planted(monkeypatch, which):
    if which == "slot_page_swapped":
        def bad(pages, block_table, b, h, n):
            P = pages.shape[2]
            t = np.arange(n)
            pid = block_table[b, np.minimum(t % P, block_table.shape[1] - 1)].astype(np.int64)
            return oracle.E5M2_TABLE[pages[pid, h, np.minimum(t // P, P - 1), :]]
        monkeypatch.setattr(A, "gather_tokens", bad)
    elif which == "scale_squared":
        monkeypatch.setattr(A, "_as_f64_scale", lambda s: float(np.float32(s)) ** 2)
    elif which == "head_map_modulo":
        orig = A.gather_tokens

        def bad(pages, block_table, b, h, n):
            return orig(pages, block_table, b, (h + 1) % pages.shape[1], n)
        monkeypatch.setattr(A, "gather_tokens", bad)
    elif which == "k_and_v_swapped":
        orig = A.decode_attention

        def bad(q, k_pages, v_pages, **kw):
            return orig(q=q, k_pages=v_pages, v_pages=k_pages, **kw)
        monkeypatch.setattr(oracle, "decode_attention", bad)


@pytest.mark.parametrize("which", ["slot_page_swapped", "scale_squared",
                                   "head_map_modulo", "k_and_v_swapped"])
def test_brute_force_catches_planted_mistakes(monkeypatch, which):
    w = make_custom([40, 21], 2, 16, 30, pool_pages=12)
    ref = np.array([[brute_force(w, b, h) for h in range(16)] for b in range(2)])
    _planted(monkeypatch, which)
    out = run_oracle(w)
    assert not np.allclose(out, ref, rtol=1e-6, equal_nan=True)


# ------------------------------- the row and split-state forms, on their own
# decode_attention_row and partial_state are pinned here against the
# pure-Python brute force (its own head map, gather and math.exp / math.fsum
# sums) at several KV heads and at group sizes 1 and 8, so a wrong head map or
# scale in either one fails; their agreement with each other is not used.

def brute_force_state(w, b, hq):
    """(m, l, o) of row (b, hq) over all its tokens with explicit loops."""
    G = w.num_q_heads // w.num_kv_heads
    h = hq // G
    n = max(0, min(int(w.context_lens[b]), w.max_pages_per_seq * w.page_size))
    kp, vp = w.pools()
    s = float(np.float32(w.scale))
    qv = [float(x) for x in w.q[b, hq, :]]
    z, vrows = [], []
    for t in range(n):
        page = int(w.block_table[b][t // w.page_size])
        slot = t % w.page_size
        kt = [_dec_bytes(int(c)) for c in kp[page, h, slot, :]]
        vrows.append([_dec_bytes(int(c)) for c in vp[page, h, slot, :]])
        z.append(s * math.fsum(qv[d] * kt[d] for d in range(w.head_dim)))
    m = max(z)
    e = [math.exp(zt - m) for zt in z]
    o = [math.fsum(e[t] * vrows[t][d] for t in range(n)) for d in range(w.head_dim)]
    return m, math.fsum(e), np.array(o)


ROW_SHAPES = [  # (context lengths, Hkv, Hq): group sizes 8 and 1, two and four KV heads
    ([23, 40], 2, 16),
    ([37, 1], 4, 4),
    ([18], 2, 2),
]


def _row_close(got, ref):
    scale = max(np.abs(ref).max(), 1e-300)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * scale)


@pytest.mark.parametrize("ctx,hkv,hq", ROW_SHAPES)
def test_decode_attention_row_matches_brute_force(ctx, hkv, hq):
    w = make_custom(ctx, hkv, hq, 40 + hq, pool_pages=sum((c + 15) // 16 for c in ctx) + 2)
    kp, vp = w.pools()
    full = run_oracle(w)
    for b in range(w.batch):
        for h in range(hq):
            row = oracle.decode_attention_row(w.q, kp, vp, w.block_table, w.context_lens,
                                              w.scale, b, h)
            ref = np.array(brute_force(w, b, h))
            _row_close(row, ref)
            _row_close(full[b, h], ref)


@pytest.mark.parametrize("ctx,hkv,hq", ROW_SHAPES)
def test_partial_state_over_all_tokens_matches_brute_force(ctx, hkv, hq):
    w = make_custom(ctx, hkv, hq, 50 + hq, pool_pages=sum((c + 15) // 16 for c in ctx) + 2)
    kp, vp = w.pools()
    G = hq // hkv
    for b in range(w.batch):
        n = int(w.context_lens[b])
        for h in range(hq):
            # The test gathers with its own head map (contiguous groups).
            K = A.gather_tokens(kp, w.block_table, b, h // G, n)
            V = A.gather_tokens(vp, w.block_table, b, h // G, n)
            m, l, o = oracle.partial_state(w.q[b, h], K, V, w.scale)
            bm, bl, bo = brute_force_state(w, b, h)
            assert abs(m - bm) <= 1e-12 * max(abs(bm), 1.0)
            assert abs(l - bl) <= 1e-12 * bl
            _row_close(o, bo)
            _row_close(oracle.merge_states([(m, l, o)]), np.array(brute_force(w, b, h)))


def _plant_row_state(monkeypatch, which):
    if which == "head_map_interleaved":
        monkeypatch.setattr(A, "_kv_head", lambda hq, Hq, Hkv: hq % Hkv)
    elif which == "scale_squared":
        monkeypatch.setattr(A, "_as_f64_scale", lambda s: float(np.float32(s)) ** 2)


@pytest.mark.parametrize("which", ["head_map_interleaved", "scale_squared"])
def test_row_pin_catches_planted_mistakes(monkeypatch, which):
    w = make_custom([23, 40], 2, 16, 56, pool_pages=6)
    kp, vp = w.pools()
    refs = {(b, h): np.array(brute_force(w, b, h)) for b in range(2) for h in range(16)}
    _plant_row_state(monkeypatch, which)
    caught = False
    for (b, h), ref in refs.items():
        row = oracle.decode_attention_row(w.q, kp, vp, w.block_table, w.context_lens, w.scale, b, h)
        caught |= not np.allclose(row, ref, rtol=1e-6)
    assert caught


def test_state_pin_catches_planted_scale(monkeypatch):
    w = make_custom([40], 2, 16, 57, pool_pages=4)
    kp, vp = w.pools()
    K = A.gather_tokens(kp, w.block_table, 0, 1, 40)
    V = A.gather_tokens(vp, w.block_table, 0, 1, 40)
    bm, bl, bo = brute_force_state(w, 0, 11)
    _plant_row_state(monkeypatch, "scale_squared")
    m, l, o = oracle.partial_state(w.q[0, 11], K, V, w.scale)
    assert abs(m - bm) > 1e-6 * max(abs(bm), 1.0)
    assert not np.allclose(oracle.merge_states([(m, l, o)]), np.array(brute_force(w, 0, 11)), rtol=1e-6)
