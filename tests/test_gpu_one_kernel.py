"""GPU parity of handles whose bounds keep every sequence in one work item.

On such a handle (one item per KV head, or at most 32 tokens per sequence)
no sequence leaves split states, so a decode step is the split kernel alone
and that kernel also writes the zero rows of empty sequences. Checked
against the float64 oracle, with empty and negative lengths spread over
many 64-sequence chunks, NaN-poisoned outputs, and graph replays that must
equal eager calls bitwise.
"""

import numpy as np
import pytest
import torch

import oracle
from tests._helpers import assert_parity, ensure_library
from workloads import make_custom
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def Xqa(**kw):
    from decode_attention_paged_e5m2_amd import Xqa as X
    return X(**kw)


def _lengths(rng, batch, hi, empty_frac):
    n = rng.integers(1, hi + 1, size=batch)
    n[rng.random(batch) < empty_frac] = 0
    return n


def _cases():
    rng = np.random.default_rng(90)
    return [
        # name, lengths, Hkv, Hq, max_pages_per_seq, max_work_items
        ("tiny B1 256", [256], 1, 8, 16, 0),
        ("700 sequences of at most 32 tokens", _lengths(rng, 700, 32, 0.2), 2, 16, 2, 0),
        ("one item per head, ragged B16", _lengths(rng, 16, 2048, 0.25), 4, 32, 128, 4),
        ("one item per head, 130 sequences", _lengths(rng, 130, 200, 0.3), 2, 8, 16, 2),
    ]


@pytest.mark.parametrize("case", range(4))
def test_one_kernel_parity_and_zero_rows(case):
    name, ctx, hkv, hq, pages, mwi = _cases()[case]
    ctx = np.asarray(ctx, dtype=np.int64)
    w = make_custom(ctx.tolist(), hkv, hq, [91, case], max_pages_per_seq=pages)
    xqa = Xqa(max_batch=w.batch, num_q_heads=hq, num_kv_heads=hkv, max_pages_per_seq=pages,
              max_work_items=mwi)
    assert xqa.info["kernels_per_step"] == 1, xqa.info
    dev = to_device(w)
    lens = dev.context_lens.clone()
    if w.batch > 1:   # a negative length is an empty sequence too
        lens[1] = -5
    lens_np = lens.cpu().numpy()
    print(f"[one-kernel] {name}: batch {w.batch}, {int((lens_np <= 0).sum())} empty, "
          f"info {xqa.info}", flush=True)

    def step(out):
        xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages, block_table=dev.block_table,
                   context_lens=lens, scale=w.scale, out=out)

    out = torch.full_like(dev.q, float("nan"))
    step(out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    kp, vp = w.pools()
    ref = oracle.decode_attention(w.q, kp, vp, w.block_table, lens_np, w.scale)
    assert_parity(got, ref, name)
    assert (got[lens_np <= 0] == 0).all()

    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_split_handles_keep_two_kernels():
    # Handles on which a sequence can span items keep the combine kernel.
    assert Xqa(max_batch=16, num_q_heads=32, num_kv_heads=4,
               max_pages_per_seq=4096).info["kernels_per_step"] == 2
    assert Xqa(max_batch=4, num_q_heads=32, num_kv_heads=4,
               max_pages_per_seq=64).info["kernels_per_step"] == 2


def test_one_kernel_multi_token_rows():
    # Two query tokens per sequence (16 rows per KV head) on a one-item-per-
    # head handle: empty sequences, a length-1 sequence whose first token
    # sees nothing, and ragged lengths, against the float64 oracle.
    rng = np.random.default_rng(93)
    ctx = rng.integers(2, 600, size=70)
    ctx[[0, 5, 64, 69]] = 0
    ctx[7] = 1
    w = make_custom(ctx.tolist(), 2, 16, [94, 0], max_pages_per_seq=40)
    xqa = Xqa(max_batch=w.batch, num_q_heads=16, num_kv_heads=2, max_pages_per_seq=40,
              max_work_items=2, max_query_tokens=2)
    assert xqa.info["kernels_per_step"] == 1
    dev = to_device(w)
    q = rng.standard_normal((w.batch, 2, 16, 128)).astype(np.float16)
    qd = torch.from_numpy(q).to(dev.q.device)
    out = torch.full_like(qd, float("nan"))
    xqa.decode(q=qd, k_pages=dev.k_pages, v_pages=dev.v_pages, block_table=dev.block_table,
               context_lens=dev.context_lens, scale=w.scale, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    kp, vp = w.pools()
    ref = oracle.decode_attention_multi(q, kp, vp, w.block_table, w.context_lens, w.scale)
    assert_parity(got, ref, "one-kernel multi-token")
    assert (got[ctx == 0] == 0).all()
    assert (got[7, 0] == 0).all()


def test_one_kernel_handle_two_stage_calls_match_decode():
    # xqa_decode_split + xqa_decode_combine stay valid on a one-kernel handle
    # (the split kernel writes every row, the combine finds nothing to merge).
    rng = np.random.default_rng(95)
    ctx = rng.integers(0, 500, size=80)
    ctx[[2, 63, 64]] = 0
    w = make_custom(ctx.tolist(), 2, 16, [96, 0], max_pages_per_seq=32)
    xqa = Xqa(max_batch=w.batch, num_q_heads=16, num_kv_heads=2, max_pages_per_seq=32,
              max_work_items=2)
    assert xqa.info["kernels_per_step"] == 1
    dev = to_device(w)
    args = dict(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages, block_table=dev.block_table,
                context_lens=dev.context_lens, scale=w.scale)
    one = xqa.decode(out=torch.full_like(dev.q, float("nan")), **args)
    two = xqa.split(out=torch.full_like(dev.q, float("nan")), **args)
    xqa.combine(context_lens=dev.context_lens, out=two)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    assert (one.float().cpu().numpy()[ctx == 0] == 0).all()
