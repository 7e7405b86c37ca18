"""The five synthetic decode workloads, plus a generic builder for test sweeps.

Each workload is a batch of sequences with one new query token each, a paged
FP8-E5M2 K/V pool laid out [num_pages, Hkv, P, D], a block table mapping each
sequence's logical pages to physical pages, and per-sequence context lengths.

Recipe (fixed here because the pages give none; the design notes list it):

* seed: ``np.random.default_rng([1000 + config_number, variant])``;
* draw order: context lengths (ragged config only) -> page permutation ->
  q [B, Hq, D] -> for each sequence in batch order: K [n, Hkv, D], V, then
  (boundary config only) the K and V outlier masks;
* q ~ N(0, 1) drawn in float32 and rounded to float16 (round to nearest even);
* K, V drawn in float32 (V optionally scaled by a std), optional outliers
  (independent Bernoulli per element, multiplied by 1000), then rounded to
  E5M2 from float32, saturating at 57344;
* pages: a seeded permutation of the pool; sequence b takes the next
  ceil(n_b / P) entries in batch order (the tiny B1 workload: identity pages);
* pool = the stated number of data pages plus one poison page (the last);
  every byte not holding a real token (tail slots, unreferenced pages, the
  poison page) is the NaN code 0x7F, and unused block-table entries point at
  the poison page.
"""

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .quantize import quantize_e4m3, quantize_e5m2, POISON_CODE

HEAD_DIM = 128
PAGE_SIZE = 16
DEFAULT_SCALE = float(np.float32(1.0 / np.sqrt(128.0)))

CONFIG_NAMES = {
    1: "tiny_b1_hkv1_ctx256",
    2: "uniform_b4_hkv4_ctx1024",
    3: "uniform_b8_hkv4_ctx16384",
    4: "ragged_b16_hkv4_ctx2048-33600",
    5: "boundary_b16_hkv4_outliers",
}

BOUNDARY_CONTEXTS = [1, 15, 16, 17, 255, 256, 257, 1023, 1024, 1025,
                     4095, 4097, 16383, 16385, 65536, 262144]


@dataclass
class Workload:
    name: str
    seed: tuple
    batch: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    page_size: int
    max_pages_per_seq: int
    num_pages: int              # data pages + 1 poison page
    poison_page: int
    context_lens: np.ndarray    # int32 [B]
    block_table: np.ndarray     # int32 [B, max_pages_per_seq]
    q: np.ndarray               # float16 [B, Hq, D]
    k_tokens: List[np.ndarray] = field(repr=False)   # uint8 [n_b, Hkv, D] per sequence
    v_tokens: List[np.ndarray] = field(repr=False)
    scale: float = DEFAULT_SCALE
    kv_format: str = "e5m2"     # byte format of k_tokens / v_tokens: "e5m2" or "e4m3"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(np.maximum(self.context_lens.astype(np.int64), 0).sum())

    @property
    def kv_bytes(self) -> int:
        """K and V bytes an exact implementation must read: 2 * Hkv * D per token."""
        return 2 * self.num_kv_heads * self.head_dim * self.total_tokens

    def token_locations(self, b: int):
        """(physical page id, slot) of every cached token of sequence b."""
        n = int(self.context_lens[b])
        t = np.arange(n)
        return self.block_table[b, t // self.page_size].astype(np.int64), t % self.page_size

    def pools(self):
        """Full K and V pools as uint8 numpy arrays [num_pages, Hkv, P, D]."""
        if len(self.k_tokens) != self.batch:
            raise ValueError("workload was built without token data")
        shape = (self.num_pages, self.num_kv_heads, self.page_size, self.head_dim)
        k = np.full(shape, POISON_CODE, dtype=np.uint8)
        v = np.full(shape, POISON_CODE, dtype=np.uint8)
        for b in range(self.batch):
            if int(self.context_lens[b]) <= 0:
                continue
            pg, slot = self.token_locations(b)
            k[pg, :, slot, :] = self.k_tokens[b]
            v[pg, :, slot, :] = self.v_tokens[b]
        return k, v


def make_custom(context_lens: Sequence[int], num_kv_heads: int, num_q_heads: int,
                seed, *, pool_pages: Optional[int] = None,
                max_pages_per_seq: Optional[int] = None, identity_pages: bool = False,
                v_std: float = 1.0, outlier_frac: float = 0.0,
                outlier_scale: float = 1000.0, scale: float = DEFAULT_SCALE,
                name: str = "custom", rng: Optional[np.random.Generator] = None,
                head_dim: int = HEAD_DIM, page_size: int = PAGE_SIZE,
                with_tokens: bool = True, kv_format: str = "e5m2") -> Workload:
    """Build a workload with the recipe above for arbitrary context lengths."""
    quantize = {"e5m2": quantize_e5m2, "e4m3": quantize_e4m3}[kv_format]
    if rng is None:
        rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64)
    B = ctx.shape[0]
    P = page_size
    pos = np.maximum(ctx, 0)
    pages_needed = (pos + P - 1) // P
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, int(pages_needed.max()) if B else 1)
    if (pages_needed > max_pages_per_seq).any():
        raise ValueError("a context does not fit max_pages_per_seq")
    used = int(pages_needed.sum())
    if pool_pages is None:
        pool_pages = max(used, 1)
    if used > pool_pages:
        raise ValueError("pool too small for the contexts")
    num_pages = pool_pages + 1
    poison = pool_pages

    if identity_pages:
        order = np.arange(pool_pages)
    else:
        order = rng.permutation(pool_pages)
    block_table = np.full((B, max_pages_per_seq), poison, dtype=np.int32)
    off = 0
    for b in range(B):
        k = int(pages_needed[b])
        block_table[b, :k] = order[off:off + k]
        off += k

    q = rng.standard_normal((B, num_q_heads, head_dim), dtype=np.float32).astype(np.float16)

    k_tokens, v_tokens = [], []
    for b in range(B if with_tokens else 0):
        n = int(pos[b])
        kf = rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32)
        vf = rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32)
        if v_std != 1.0:
            vf *= np.float32(v_std)
        if outlier_frac > 0.0:
            mk = rng.random((n, num_kv_heads, head_dim)) < outlier_frac
            mv = rng.random((n, num_kv_heads, head_dim)) < outlier_frac
            kf[mk] *= np.float32(outlier_scale)
            vf[mv] *= np.float32(outlier_scale)
        k_tokens.append(quantize(kf))
        v_tokens.append(quantize(vf))

    return Workload(
        name=name, seed=tuple(np.atleast_1d(seed).tolist()) if seed is not None else (),
        batch=B, num_kv_heads=num_kv_heads, num_q_heads=num_q_heads,
        head_dim=head_dim, page_size=P, max_pages_per_seq=int(max_pages_per_seq),
        num_pages=num_pages, poison_page=poison,
        context_lens=ctx.astype(np.int32), block_table=block_table, q=q,
        k_tokens=k_tokens, v_tokens=v_tokens, scale=float(np.float32(scale)), kv_format=kv_format)


def make_config(index: int, variant: int = 0, with_tokens: bool = True,
                kv_format: str = "e5m2") -> Workload:
    """Workload 1..5 of CONFIG_NAMES (recipe in the module docstring),
    deterministic in (index, variant).

    ``with_tokens=False`` stops after the block table and q (same draws), for
    callers that only need the shapes, lengths and page assignment.
    """
    seed = [1000 + index, variant]
    rng = np.random.default_rng(seed)
    name = f"{CONFIG_NAMES[index]}_v{variant}"
    kw = dict(name=name, rng=rng, with_tokens=with_tokens, kv_format=kv_format)
    if index == 1:
        return make_custom([256], 1, 8, seed, pool_pages=16, max_pages_per_seq=16,
                           identity_pages=True, **kw)
    if index == 2:
        return make_custom([1024] * 4, 4, 32, seed, pool_pages=256, max_pages_per_seq=64, **kw)
    if index == 3:
        return make_custom([16384] * 8, 4, 32, seed, pool_pages=8 * 16384,
                           max_pages_per_seq=16384, v_std=0.5, **kw)
    if index == 4:
        ctx = rng.integers(2048, 33601, size=16)
        return make_custom(ctx.tolist(), 4, 32, seed, pool_pages=16 * 16384,
                           max_pages_per_seq=16384, **kw)
    if index == 5:
        return make_custom(BOUNDARY_CONTEXTS, 4, 32, seed, pool_pages=16 * 16384,
                           max_pages_per_seq=16384, outlier_frac=0.01, **kw)
    raise ValueError("config index must be 1..5")
