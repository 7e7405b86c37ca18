"""Float64 decode attention over a selected subset of each sequence's pages
(test infrastructure only).

The page "[Kernel][WIP] Follow up FlashNext batch HC fusion and QSA route
audit" (section Test Result) describes sparse decode attention in which a
planner chooses, per query, which KV pages to attend over (its "Page4
selection", "per-query logical-order plan", "index expansion" and causal-tail
items). It publishes neither the selection rule nor the planner's data, so
the selection is an input here and the operation is the attention over the
tokens it names. Readings taken where the page is silent:

* The selection is per sequence (shared by all its KV heads and query heads):
  ``page_select[b, 0:select_counts[b]]`` lists logical page indices of
  sequence b (index p covers tokens p*P .. p*P + P - 1).
* Entries are taken in list order. An entry is kept iff it names a page the
  sequence uses (0 <= p < ceil(n / P), n as for plain decode) and is greater
  than every entry kept before it; any other entry (out of range, repeated,
  or out of ascending order) is skipped. Counts outside [0, S] are clamped.
* The query attends over the tokens t < n of the kept pages, with the same
  scores, softmax and weighted sum as plain decode. No kept token gives a
  zero row.

With every page selected in order this is exactly ``decode_attention``.
"""

import numpy as np

from .e5m2 import E5M2_TABLE


def kept_pages(page_select, select_counts, n: int, P: int, b: int) -> list:
    """The logical pages of sequence b that the selection keeps, in order."""
    S = page_select.shape[1]
    count = min(max(int(select_counts[b]), 0), S)
    used = -(-n // P) if n > 0 else 0
    kept = []
    for j in range(count):
        p = int(page_select[b, j])
        if 0 <= p < used and (not kept or p > kept[-1]):
            kept.append(p)
    return kept


def selected_tokens(page_select, select_counts, n: int, P: int, b: int) -> np.ndarray:
    """Logical token indices t < n of the kept pages, in page order."""
    toks = [t for p in kept_pages(page_select, select_counts, n, P, b)
            for t in range(p * P, min((p + 1) * P, n))]
    return np.asarray(toks, dtype=np.int64)


def decode_attention_pages(q, k_pages, v_pages, block_table, context_lens, page_select,
                           select_counts, scale) -> np.ndarray:
    """Decode attention restricted to the selected pages: float64 [B, Hq, D].

    Shapes: q [B, Hq, D]; k_pages / v_pages uint8 [num_pages, Hkv, P, D];
    block_table int [B, max_pages_per_seq]; context_lens int [B];
    page_select int [B, S]; select_counts int [B].
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    P = k_pages.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    s64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    cap = block_table.shape[1] * P
    for b in range(B):
        n = max(0, min(int(context_lens[b]), cap))
        t = selected_tokens(page_select, select_counts, n, P, b)
        if t.size == 0:
            continue
        phys = block_table[b, t // P].astype(np.int64)
        for h in range(Hkv):
            K = E5M2_TABLE[k_pages[phys, h, t % P, :]]
            V = E5M2_TABLE[v_pages[phys, h, t % P, :]]
            Qg = np.asarray(q[b, h * G:(h + 1) * G, :], dtype=np.float64)
            Z = s64 * (Qg @ K.T)
            W = np.exp(Z - Z.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G, :] = (W @ V) / W.sum(axis=1, keepdims=True)
    return out
