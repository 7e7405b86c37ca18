"""GPU parity of multi-token decode (xqa_decode_multi) against the float64 oracle.

M new query tokens per sequence, causal among themselves; the G * M query
rows of a KV head share the matrix-core tile. Same tolerance as single-token
decode; exact zeros for query rows that see no token.
"""

import numpy as np
import pytest
import torch

import oracle
from tests._helpers import assert_parity, ensure_library
from workloads import make_config, make_custom
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def Xqa(**kw):
    from decode_attention_paged_e5m2_amd import Xqa as X
    return X(**kw)


def _q_multi(w, M, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((w.batch, M, w.num_q_heads, w.head_dim)).astype(np.float16)


def _run(w, q, xqa=None, dev=None, max_work_items=0):
    M = q.shape[1]
    if dev is None:
        dev = to_device(w)
    if xqa is None:
        xqa = Xqa(max_batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                  max_pages_per_seq=w.max_pages_per_seq, max_work_items=max_work_items,
                  max_query_tokens=M)
    qd = torch.from_numpy(q).to(dev.q.device)
    out = xqa.decode(q=qd, k_pages=dev.k_pages, v_pages=dev.v_pages, block_table=dev.block_table,
                     context_lens=dev.context_lens, scale=w.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), xqa, dev


def _ref(w, q):
    kp, vp = w.pools()
    return oracle.decode_attention_multi(q, kp, vp, w.block_table, w.context_lens, w.scale)


@pytest.mark.parametrize("hkv,hq,M", [(4, 32, 2), (8, 32, 4), (2, 2, 16), (1, 4, 4), (4, 16, 3)])
def test_multi_sweep(hkv, hq, M):
    # Lengths below, at and just above M, around 32-token blocks, and long.
    lens = [1, M - 1 if M > 1 else 2, M, M + 1, 31, 32, 33, 47, 300, 2049, 0, 5000]
    w = make_custom(lens, hkv, hq, [61, hkv, hq, M], pool_pages=800)
    q = _q_multi(w, M, 62 + M)
    out, _, _ = _run(w, q)
    ref = _ref(w, q)
    assert_parity(out, ref, f"multi hkv={hkv} hq={hq} M={M}")
    n = np.maximum(np.asarray(lens), 0)
    for b in range(len(lens)):
        for j in range(M):
            if n[b] - M + j < 0:
                assert (out[b, j] == 0).all(), (b, j)


def test_one_query_token_is_bitwise_the_single_token_decode():
    w = make_custom([1, 17, 300, 2049, 0], 4, 32, [63, 0], pool_pages=400)
    dev = to_device(w)
    xqa = Xqa(max_batch=w.batch, num_q_heads=32, num_kv_heads=4,
              max_pages_per_seq=w.max_pages_per_seq, max_query_tokens=2)
    single = xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                        block_table=dev.block_table, context_lens=dev.context_lens, scale=w.scale)
    multi = xqa.decode(q=dev.q.unsqueeze(1).contiguous(), k_pages=dev.k_pages,
                       v_pages=dev.v_pages, block_table=dev.block_table,
                       context_lens=dev.context_lens, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(single.view(torch.int16), multi[:, 0].view(torch.int16))


@pytest.mark.parametrize("per_head", [1, 3, 7])
def test_multi_work_item_boundaries(per_head):
    # Few work items per head: the masked last tokens of a sequence fall on
    # item and block boundaries and on items shared by several sequences.
    lens = [33, 64, 65, 95, 96, 97, 255, 256, 257, 1000, 4, 3]
    M = 4
    w = make_custom(lens, 2, 8, [64, per_head], pool_pages=200)
    q = _q_multi(w, M, 65)
    out, xqa, _ = _run(w, q, max_work_items=2 * per_head)
    S, items = xqa.plan(w.context_lens)
    assert_parity(out, _ref(w, q), f"multi boundaries per_head={per_head} S={S} items={items}")


def test_multi_full_size_ragged_b16_two_tokens():
    # The ragged B16 shape with two tokens per sequence: 8 heads x 2 tokens
    # fill the 16-row tile.
    w = make_config(4)
    q = _q_multi(w, 2, 66)
    out, _, _ = _run(w, q)
    assert_parity(out, _ref(w, q), "cfg4 M=2")


def test_multi_graph_replays_equal_eager():
    ws = [make_custom([700, 33, 5, 2100], 4, 16, [67, v], pool_pages=300, max_pages_per_seq=140)
          for v in range(2)]
    M = 3
    devs = [to_device(w) for w in ws]
    xqa = Xqa(max_batch=4, num_q_heads=16, num_kv_heads=4, max_pages_per_seq=140,
              max_query_tokens=M)
    qs = [torch.from_numpy(_q_multi(w, M, 68 + i)).to("cuda:0") for i, w in enumerate(ws)]
    q_buf = torch.empty_like(qs[0])
    lens = torch.empty_like(devs[0].context_lens)
    bt = torch.empty_like(devs[0].block_table)
    out = torch.empty_like(qs[0])

    def step(i):
        xqa.decode(q=q_buf, k_pages=devs[i].k_pages, v_pages=devs[i].v_pages, block_table=bt,
                   context_lens=lens, scale=ws[0].scale, out=out)

    def load(i):
        q_buf.copy_(qs[i])
        lens.copy_(devs[i].context_lens)
        bt.copy_(devs[i].block_table)

    eager = []
    for i in range(2):
        load(i)
        step(i)
        torch.cuda.synchronize()
        eager.append(out.clone())
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for r in range(8):
        i = r % 2
        load(i)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graphs[i].replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[i].view(torch.int16)), f"replay {r}"
    for i in range(2):
        assert_parity(eager[i].float().cpu().numpy(), _ref(ws[i], qs[i].cpu().numpy()), f"graph {i}")
