"""Float64 paged grouped-query decode attention (test infrastructure only).

Operation (page "[Kernel][SM70] Pipeline batched E5M2 XQA decode", sections
Purpose and Pending work and gates: batched XQA decode over an FP8 E5M2 paged
KV cache with randomized physical pages). For every sequence b and query head
hq, with G = Hq / Hkv query heads per KV head:

    h   = hq // G                      (contiguous head groups; a reading)
    n   = min(context_lens[b], max_pages_per_seq * P)
    for t in 0..n-1:  page = block_table[b, t // P], slot = t % P
        k_t = dec(k_pages[page, h, slot, :]),  v_t = dec(v_pages[page, h, slot, :])
        z_t = scale * sum_d q[b, hq, d] * k_t[d]
    out[b, hq, :] = sum_t exp(z_t - max z) v_t / sum_t exp(z_t - max z)
    n <= 0 gives a zero row.

Readings (the pages are silent on these): K and V pools are laid out
[num_pages, Hkv, P, D]; scale multiplies the raw dot product and is an fp32
value; there are no per-tensor dequantisation scales; every cached token
t < n attends (one query token needs no causal mask); slots >= n of the last
page and pages not referenced never enter the result.

Everything is float64. ``partial_state`` / ``merge_states`` restate the same
softmax over a subset of the tokens and its exact log-sum-exp merge; merging
the states of any partition of 0..n-1 gives ``decode_attention_row`` up to
rounding, which is what pins a split-context implementation.
"""

import numpy as np

from .e5m2 import E5M2_TABLE


def _as_f64_scale(scale) -> float:
    # The scale crosses the boundary as an fp32 value.
    return float(np.float32(scale))


def gather_tokens(pages: np.ndarray, block_table: np.ndarray, b: int, h: int, n: int) -> np.ndarray:
    """Decoded rows [n, D] (float64) of KV head h for sequence b, in logical token order."""
    P = pages.shape[2]
    t = np.arange(n)
    page_ids = block_table[b, t // P].astype(np.int64)
    slots = t % P
    codes = pages[page_ids, h, slots, :]
    return E5M2_TABLE[codes]


def _kv_head(hq: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head hq: contiguous groups of G = Hq / Hkv (a reading)."""
    return hq // (Hq // Hkv)


def _effective_len(context_lens, block_table, P, b) -> int:
    n = int(context_lens[b])
    return max(0, min(n, block_table.shape[1] * P))


def decode_attention_row(q, k_pages, v_pages, block_table, context_lens, scale, b, hq) -> np.ndarray:
    """Output row out[b, hq, :] as float64."""
    Hq = q.shape[1]
    Hkv = k_pages.shape[1]
    P = k_pages.shape[2]
    D = k_pages.shape[3]
    h = _kv_head(hq, Hq, Hkv)
    n = _effective_len(context_lens, block_table, P, b)
    if n == 0:
        return np.zeros(D, dtype=np.float64)
    K = gather_tokens(k_pages, block_table, b, h, n)
    V = gather_tokens(v_pages, block_table, b, h, n)
    qv = np.asarray(q[b, hq, :], dtype=np.float64)
    z = _as_f64_scale(scale) * (K @ qv)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def decode_attention(q, k_pages, v_pages, block_table, context_lens, scale) -> np.ndarray:
    """The full operation: float64 array [B, Hq, D].

    Shapes: q [B, Hq, D] (float16 values), k_pages / v_pages uint8
    [num_pages, Hkv, P, D], block_table int [B, max_pages_per_seq],
    context_lens int [B].
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    P = k_pages.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if k_pages.shape != v_pages.shape or k_pages.shape[3] != D:
        raise ValueError("page pools must be [num_pages, Hkv, P, D] and agree")
    G = Hq // Hkv
    s64 = _as_f64_scale(scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = _effective_len(context_lens, block_table, P, b)
        if n == 0:
            continue
        for h in range(Hkv):
            K = gather_tokens(k_pages, block_table, b, h, n)
            V = gather_tokens(v_pages, block_table, b, h, n)
            Qg = np.asarray(q[b, h * G:(h + 1) * G, :], dtype=np.float64)   # [G, D]
            Z = s64 * (Qg @ K.T)                                             # [G, n]
            W = np.exp(Z - Z.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G, :] = (W @ V) / W.sum(axis=1, keepdims=True)
    return out


def partial_state(qv, K, V, scale):
    """Softmax state of one query row over a subset of tokens.

    Returns (m, l, o): m = max_t z_t, l = sum_t exp(z_t - m),
    o = sum_t exp(z_t - m) v_t (unnormalised), with z_t = scale * q . k_t.
    An empty subset gives (-inf, 0, 0).
    """
    qv = np.asarray(qv, dtype=np.float64)
    D = qv.shape[0]
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(D, dtype=np.float64)
    z = _as_f64_scale(scale) * (K @ qv)
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ V


def merge_states(states):
    """Exact log-sum-exp merge of partial states, in the order given.

    M = max_s m_s; L = sum_s l_s exp(m_s - M); out = sum_s exp(m_s - M) o_s / L.
    """
    ms = np.array([s[0] for s in states], dtype=np.float64)
    M = ms.max()
    L = 0.0
    acc = np.zeros_like(np.asarray(states[0][2], dtype=np.float64))
    for m, l, o in states:
        if m == -np.inf:
            continue
        f = np.exp(m - M)
        L += l * f
        acc = acc + f * np.asarray(o, dtype=np.float64)
    return acc / L


def decode_attention_multi(q, k_pages, v_pages, block_table, context_lens, scale) -> np.ndarray:
    """Several new query tokens per sequence, causal among themselves: float64 [B, M, Hq, D].

    q is [B, M, Hq, D]. Reading taken (the pages name multi-token rows but do
    not define them): n = min(context_lens[b], capacity) counts the M new
    tokens, so query token j sits at position n - M + j and sees tokens
    0 .. n - M + j, each through the same paged gather as a single query.
    A query that sees no token (n - M + j < 0) gives a zero row.
    """
    q = np.asarray(q)
    B, M, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    P = k_pages.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    s64 = _as_f64_scale(scale)
    out = np.zeros((B, M, Hq, D), dtype=np.float64)
    for b in range(B):
        n = _effective_len(context_lens, block_table, P, b)
        for j in range(M):
            visible = n - M + j + 1
            if visible <= 0:
                continue
            for h in range(Hkv):
                K = gather_tokens(k_pages, block_table, b, h, visible)
                V = gather_tokens(v_pages, block_table, b, h, visible)
                Qg = np.asarray(q[b, j, h * G:(h + 1) * G, :], dtype=np.float64)   # [G, D]
                Z = s64 * (Qg @ K.T)
                W = np.exp(Z - Z.max(axis=1, keepdims=True))
                out[b, j, h * G:(h + 1) * G, :] = (W @ V) / W.sum(axis=1, keepdims=True)
    return out


def decode_attention_fp8(q, k_pages, v_pages, block_table, context_lens, scale, *,
                         kv_format="e5m2", k_scale=1.0, v_scale=1.0) -> np.ndarray:
    """Decode over an FP8 cache with per-tensor dequantisation scales: float64.

    q is [B, Hq, D] (one query token per sequence) or [B, M, Hq, D] (M tokens,
    causal as in decode_attention_multi); the output has q's shape. kv_format
    is "e5m2" or "e4m3"; the cached K and V values are k_scale * dec(code) and
    v_scale * dec(code) (k_scale and v_scale cross the boundary as fp32).
    Reading taken: one scale per tensor (all pages, heads and tokens), as
    the "per-tensor scales" variant names.
    """
    from .e4m3 import E4M3_TABLE
    table = {"e5m2": E5M2_TABLE, "e4m3": E4M3_TABLE}[kv_format]
    q = np.asarray(q)
    single = q.ndim == 3
    q4 = q[:, None] if single else q
    B, M, Hq, D = q4.shape
    Hkv = k_pages.shape[1]
    P = k_pages.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    s64 = _as_f64_scale(scale)
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    out = np.zeros((B, M, Hq, D), dtype=np.float64)
    for b in range(B):
        n = _effective_len(context_lens, block_table, P, b)
        for j in range(M):
            visible = n - M + j + 1
            if visible <= 0:
                continue
            t = np.arange(visible)
            pages = block_table[b, t // P].astype(np.int64)
            for h in range(Hkv):
                K = ks * table[k_pages[pages, h, t % P, :]]
                V = vs * table[v_pages[pages, h, t % P, :]]
                Qg = np.asarray(q4[b, j, h * G:(h + 1) * G, :], dtype=np.float64)
                Z = s64 * (Qg @ K.T)
                W = np.exp(Z - Z.max(axis=1, keepdims=True))
                out[b, j, h * G:(h + 1) * G, :] = (W @ V) / W.sum(axis=1, keepdims=True)
    return out[:, 0] if single else out
