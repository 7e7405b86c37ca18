"""GPU tests at the documented maximum sizes: a sequence of 2^24 tokens
(max_pages_per_seq * 16), also through page-subset decode with a selection
row of 2^20 pages, and a batch of 65536 sequences.

The longest sequence is checked through a closed form instead of the
element-wise oracle: with every K row the same code all scores are equal,
the weights are exactly 1, and each output is the plain mean of V over the
sequence, which the residue pattern of V gives exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.e5m2 import E5M2_TABLE
from tests._helpers import assert_parity, ensure_library
from workloads import make_custom, make_selection
from workloads.device import to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def Xqa(**kw):
    from decode_attention_paged_e5m2_amd import Xqa as X
    return X(**kw)


# V codes of 1.0, 1.25, 1.5, 1.75 and 2.0: token t, head-dim d holds
# CODES[(t + d) % 5], so every mean over a token range is a count of residues.
CODES = np.array([0x3C, 0x3D, 0x3E, 0x3F, 0x40], dtype=np.int64)


def _mean_of_pattern(n, d):
    # Tokens 0..n-1 in column d: residue (t + d) % 5 occurs floor or ceil n/5 times.
    r = (np.arange(5) - d) % 5            # token residues t % 5 that give code index k
    counts = np.array([(n - rr + 4) // 5 if rr < n else 0 for rr in r])
    return float((counts * E5M2_TABLE[CODES]).sum() / n)


def test_longest_sequence_2_pow_24_tokens():
    n = 1 << 24                      # 16,777,216 tokens = 1,048,576 pages
    pages = n // 16
    hkv, hq = 1, 8
    dev = torch.device("cuda", 0)
    print(f"[limits] building a {n}-token sequence ({pages} pages)", flush=True)
    k = torch.full((pages, hkv, 16, 128), 0x3C, dtype=torch.uint8, device=dev)
    t = torch.arange(n, device=dev, dtype=torch.int32).view(pages, 1, 16, 1)
    d = torch.arange(128, device=dev, dtype=torch.int32).view(1, 1, 1, 128)
    codes = torch.tensor(CODES, dtype=torch.uint8, device=dev)
    v = codes[(t + d) % 5]
    del t, d
    bt = torch.arange(pages, dtype=torch.int32, device=dev).view(1, pages)
    q = torch.randn((1, hq, 128), generator=torch.Generator().manual_seed(9)).half().to(dev)
    out = torch.empty_like(q)
    xqa = Xqa(max_batch=1, num_q_heads=hq, num_kv_heads=hkv, max_pages_per_seq=pages)
    S, items = xqa.plan(np.array([n], dtype=np.int32))
    for length in (n, n - 5, 1000003):
        lens = torch.tensor([length], dtype=torch.int32, device=dev)
        xqa.decode(q=q, k_pages=k, v_pages=v, block_table=bt, context_lens=lens, scale=0.088,
                   out=out)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()[0]
        want = np.array([_mean_of_pattern(length, dd) for dd in range(128)])
        err = np.abs(got - want[None, :]).max()
        print(f"[limits] n={length} split={S} items={items} max|err|={err:.2e}", flush=True)
        # fp16 output rounding of values in [1, 2] is at most 2^-11; the fp32
        # sums over up to 2^24 tokens add far less than 1e-4.
        assert err <= 2.0 ** -11 + 1e-4
    xqa.close()

    # Page-subset decode over the same sequence: a selection row of 2^20
    # pages (1024 tiles of the selection kernel). Every page in order is
    # plain decode bit for bit; every third page plus the partial last one
    # is the mean of the pattern over the tokens those pages hold.
    xqa_p = Xqa(max_batch=1, num_q_heads=hq, num_kv_heads=hkv, max_pages_per_seq=pages,
                max_selected_pages=pages)
    length = n - 5
    lens = torch.tensor([length], dtype=torch.int32, device=dev)
    every = torch.arange(pages, dtype=torch.int32, device=dev).view(1, pages)
    plain = xqa_p.decode(q=q, k_pages=k, v_pages=v, block_table=bt, context_lens=lens, scale=0.088)
    sub = xqa_p.decode_pages(q=q, k_pages=k, v_pages=v, block_table=bt, context_lens=lens,
                             page_select=every,
                             select_counts=torch.tensor([pages], dtype=torch.int32, device=dev),
                             scale=0.088)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), sub.view(torch.int16))
    chosen = np.append(np.arange(0, pages - 1, 3), pages - 1)
    row = torch.full((1, pages), -1, dtype=torch.int32, device=dev)
    row[0, :chosen.size] = torch.from_numpy(chosen.astype(np.int32)).to(dev)
    sub = xqa_p.decode_pages(q=q, k_pages=k, v_pages=v, block_table=bt, context_lens=lens,
                             page_select=row,
                             select_counts=torch.tensor([chosen.size], dtype=torch.int32, device=dev),
                             scale=0.088)
    torch.cuda.synchronize()
    toks = (16 * chosen[:, None] + np.arange(16)[None, :]).ravel()
    toks = toks[toks < length]
    hist = np.bincount(toks % 5, minlength=5)            # tokens with t % 5 == r
    vals = E5M2_TABLE[CODES]
    want = np.array([(hist * vals[(np.arange(5) + dd) % 5]).sum() / toks.size for dd in range(128)])
    err = np.abs(sub.float().cpu().numpy()[0] - want[None, :]).max()
    print(f"[limits] page subset: {chosen.size} of {pages} pages, {toks.size} tokens, "
          f"max|err|={err:.2e}", flush=True)
    assert err <= 2.0 ** -11 + 1e-4
    xqa_p.close()


def test_largest_batch_65536_sequences():
    rng = np.random.default_rng(81)
    B = 65536
    lens = rng.integers(0, 40, size=B)
    lens[::97] = 0
    w = make_custom(lens.tolist(), 1, 4, [82, 0])
    print(f"[limits] batch {B}, {int(lens.sum())} tokens", flush=True)
    dev = to_device(w)
    xqa = Xqa(max_batch=B, num_q_heads=4, num_kv_heads=1, max_pages_per_seq=w.max_pages_per_seq)
    out = xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                     block_table=dev.block_table, context_lens=dev.context_lens, scale=w.scale)
    torch.cuda.synchronize()
    kp, vp = w.pools()
    ref = oracle.decode_attention(w.q, kp, vp, w.block_table, w.context_lens, w.scale)
    got = out.float().cpu().numpy()
    assert_parity(got, ref, "batch 65536")
    assert (got[lens == 0] == 0).all()
    xqa.close()

    # Page-subset decode over the same batch: 65536 selection workgroups.
    sel, counts = make_selection(lens.tolist(), w.max_pages_per_seq, 0.5, [83], messy=True)
    xqa = Xqa(max_batch=B, num_q_heads=4, num_kv_heads=1, max_pages_per_seq=w.max_pages_per_seq,
              max_selected_pages=w.max_pages_per_seq)
    out = xqa.decode_pages(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                           block_table=dev.block_table, context_lens=dev.context_lens,
                           page_select=torch.from_numpy(sel).cuda(),
                           select_counts=torch.from_numpy(counts).cuda(), scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_pages(w.q, kp, vp, w.block_table, w.context_lens, sel, counts,
                                        w.scale)
    assert_parity(out.float().cpu().numpy(), ref, "batch 65536, page subsets")
    xqa.close()
