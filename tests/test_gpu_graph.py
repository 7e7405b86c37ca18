"""hipGraph capture of the decode step: replays with changed input contents
and a poisoned output must be bitwise equal to eager calls."""

import numpy as np
import pytest
import torch

from tests._helpers import ensure_library
from workloads import make_config, make_custom
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def test_graph_replay_changed_inputs_poisoned_output():
    from decode_attention_paged_e5m2_amd import Xqa
    variants = [make_custom(ctx, 2, 16, [60, i], pool_pages=400, max_pages_per_seq=128)
                for i, ctx in enumerate([[100, 2000, 5, 900], [2047, 1, 33, 1500],
                                         [64, 64, 64, 64], [0, 1999, 700, 17]])]
    devs = [to_device(w) for w in variants]
    xqa = Xqa(max_batch=4, num_q_heads=16, num_kv_heads=2, max_pages_per_seq=128)
    # eager results per variant
    eager = []
    for w, d in zip(variants, devs):
        o = xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                       context_lens=d.context_lens, scale=w.scale)
        eager.append(o.clone())
    torch.cuda.synchronize()

    # static buffers the graph reads; pools shared by copying each variant's in
    s_q = devs[0].q.clone()
    s_bt = devs[0].block_table.clone()
    s_len = devs[0].context_lens.clone()
    s_k = devs[0].k_pages.clone()
    s_v = devs[0].v_pages.clone()
    s_out = torch.empty_like(s_q)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        xqa.decode(q=s_q, k_pages=s_k, v_pages=s_v, block_table=s_bt, context_lens=s_len,
                   scale=variants[0].scale, out=s_out)
    torch.cuda.current_stream().wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xqa.decode(q=s_q, k_pages=s_k, v_pages=s_v, block_table=s_bt, context_lens=s_len,
                   scale=variants[0].scale, out=s_out)
    torch.cuda.synchronize()

    for cycle in range(64):
        i = cycle % len(variants)
        d = devs[i]
        s_q.copy_(d.q)
        s_bt.copy_(d.block_table)
        s_len.copy_(d.context_lens)
        s_k.copy_(d.k_pages)
        s_v.copy_(d.v_pages)
        s_out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s_out.view(torch.int16), eager[i].view(torch.int16)), f"cycle {cycle}"
        if cycle % 16 == 0:
            print(f"[graph] cycle {cycle} ok", flush=True)


def test_graph_replay_config4_variants():
    from decode_attention_paged_e5m2_amd import Xqa
    ws = [make_config(4, v) for v in range(2)]
    devs = [to_device(w) for w in ws]
    xqa = Xqa(max_batch=16, num_q_heads=32, num_kv_heads=4, max_pages_per_seq=16384)
    graphs, outs, eager = [], [], []
    for w, d in zip(ws, devs):
        eager.append(xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages,
                                block_table=d.block_table, context_lens=d.context_lens,
                                scale=w.scale).clone())
    torch.cuda.synchronize()
    for w, d in zip(ws, devs):
        o = torch.empty_like(d.q)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                       context_lens=d.context_lens, scale=w.scale, out=o)
        graphs.append(g)
        outs.append(o)
    torch.cuda.synchronize()
    for cycle in range(8):
        i = cycle % 2
        outs[i].fill_(float("nan"))
        graphs[i].replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), f"cycle {cycle}"
