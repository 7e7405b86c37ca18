"""Seeded page selections for page-subset decode (inputs only, no arithmetic).

``make_selection`` draws, for every sequence, a subset of the logical pages
its context uses: each page independently with probability ``frac`` (the
sequence's last page always, so the partial tail page is exercised), listed
in ascending order. ``messy=True`` also plants entries the contract says are
skipped: out-of-range indices (negative or past the last used page),
repeats and descending entries. Rows are padded with -1 to the stride.
"""

from typing import Optional, Sequence, Tuple

import numpy as np


def make_selection(context_lens: Sequence[int], stride: int, frac: float, seed, *,
                   page_size: int = 16, messy: bool = False,
                   rng: Optional[np.random.Generator] = None) -> Tuple[np.ndarray, np.ndarray]:
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    B = lens.shape[0]
    sel = np.full((B, stride), -1, dtype=np.int32)
    counts = np.zeros(B, dtype=np.int32)
    for b in range(B):
        used = int(-(-max(int(lens[b]), 0) // page_size))
        if used == 0:
            picks = np.zeros(0, dtype=np.int64)
        else:
            picks = np.flatnonzero(rng.random(used) < frac)
            if picks.size == 0 or picks[-1] != used - 1:
                picks = np.append(picks, used - 1)
        row = list(picks)
        if messy:
            junk = [-1 - int(rng.integers(0, 4)), used + int(rng.integers(0, 4))]
            if row:
                junk += [int(row[int(rng.integers(0, len(row)))]),          # a repeat
                         int(rng.integers(0, row[-1] + 1))]                 # may descend
            for x in junk:
                row.insert(int(rng.integers(0, len(row) + 1)), x)
        row = row[:stride]
        sel[b, :len(row)] = row
        counts[b] = len(row)
    return sel, counts
