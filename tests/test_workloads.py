"""Invariants of the seeded input generator (CPU only).

A generator bug can select pages a sequence does not own (the page
"[Kernel][WIP] Follow up FlashNext batch HC fusion and QSA route audit",
section Test Result, reports exactly such a benchmark-generator defect), so
the generator gets its own checks before any kernel is compared with it.
"""

import numpy as np
import pytest

from workloads import make_config, make_custom, POISON_CODE, CONFIG_NAMES
from workloads.configs import BOUNDARY_CONTEXTS


def check_block_table(w):
    P = w.page_size
    seen = []
    for b in range(w.batch):
        n = max(int(w.context_lens[b]), 0)
        k = (n + P - 1) // P
        row = w.block_table[b]
        assert (row[k:] == w.poison_page).all()
        assert (row[:k] >= 0).all() and (row[:k] < w.poison_page).all()
        seen.append(row[:k])
    allp = np.concatenate(seen) if seen else np.zeros(0)
    assert len(np.unique(allp)) == len(allp), "a physical page is shared"


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_small_configs_invariants(idx):
    w = make_config(idx)
    check_block_table(w)
    assert w.q.dtype == np.float16 and w.q.shape == (w.batch, w.num_q_heads, 128)
    assert w.block_table.dtype == np.int32 and w.context_lens.dtype == np.int32
    for b in range(w.batch):
        n = int(w.context_lens[b])
        for arr in (w.k_tokens[b], w.v_tokens[b]):
            assert arr.shape == (n, w.num_kv_heads, 128) and arr.dtype == np.uint8
            assert (((arr >> 2) & 31) != 31).all(), "generator emitted inf/NaN"


def test_config_shapes():
    expect = {1: (1, 1, 8, 16, 17), 2: (4, 4, 32, 64, 257),
              3: (8, 4, 32, 16384, 8 * 16384 + 1), 4: (16, 4, 32, 16384, 16 * 16384 + 1),
              5: (16, 4, 32, 16384, 16 * 16384 + 1)}
    for idx, (B, hkv, hq, mp, npg) in expect.items():
        w = make_config(idx, with_tokens=False)
        assert (w.batch, w.num_kv_heads, w.num_q_heads, w.max_pages_per_seq, w.num_pages) == \
            (B, hkv, hq, mp, npg), idx
        assert w.name == f"{CONFIG_NAMES[idx]}_v0"
        check_block_table(w)
    assert make_config(1, with_tokens=False).context_lens.tolist() == [256]
    assert (make_config(1, with_tokens=False).block_table[0] == np.arange(16)).all()
    assert make_config(5, with_tokens=False).context_lens.tolist() == BOUNDARY_CONTEXTS
    c4 = make_config(4, with_tokens=False).context_lens
    assert c4.min() >= 2048 and c4.max() <= 33600


def test_ragged_lengths_differ_by_variant_and_are_deterministic():
    a = make_config(4, 0, with_tokens=False).context_lens
    b = make_config(4, 0, with_tokens=False).context_lens
    c = make_config(4, 1, with_tokens=False).context_lens
    assert (a == b).all() and not (a == c).all()


def test_metadata_only_matches_full_generation():
    full = make_config(2)
    meta = make_config(2, with_tokens=False)
    assert (full.block_table == meta.block_table).all()
    assert (full.q == meta.q).all()


def test_pool_poison_layout():
    w = make_custom([1, 15, 16, 17, 40], 2, 16, 5, pool_pages=20, max_pages_per_seq=3)
    kp, vp = w.pools()
    ref = set()
    for b in range(w.batch):
        n = int(w.context_lens[b])
        pg, slot = w.token_locations(b)
        assert (kp[pg, :, slot, :] == w.k_tokens[b]).all()
        assert (vp[pg, :, slot, :] == w.v_tokens[b]).all()
        # tail slots of the last page are poison
        if n % 16:
            last = w.block_table[b, n // 16]
            assert (kp[last, :, n % 16:, :] == POISON_CODE).all()
            assert (vp[last, :, n % 16:, :] == POISON_CODE).all()
        ref.update(pg.tolist())
    unref = [p for p in range(w.num_pages) if p not in ref]
    assert w.poison_page in unref
    assert (kp[unref] == POISON_CODE).all() and (vp[unref] == POISON_CODE).all()


def test_outliers_present_in_boundary_recipe():
    w = make_custom([4000], 1, 8, 6, outlier_frac=0.01)
    from oracle import decode_e5m2   # decoding bytes to check the draw, not the method
    v = np.abs(decode_e5m2(w.k_tokens[0]))
    frac = (v > 100).mean()
    assert 0.005 < frac < 0.015
