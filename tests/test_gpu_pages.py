"""GPU parity of page-subset decode (xqa_decode_pages) through the C ABI.

Against the float64 oracle (``oracle.decode_attention_pages``) under the
stated tolerance, plus bitwise checks the construction fixes: selecting every
page in order is plain decode, pages left out never matter, graph replays
with changed selections equal eager calls.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests._helpers import assert_parity, ensure_library
from workloads import make_config, make_custom, make_selection
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def Xqa(**kw):
    from decode_attention_paged_e5m2_amd import Xqa as X
    return X(**kw)


def handle_for(w, stride=None, **kw):
    return Xqa(max_batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
               max_pages_per_seq=w.max_pages_per_seq,
               max_selected_pages=stride or w.max_pages_per_seq, **kw)


def run_pages(xqa, w, d, sel, counts, out=None):
    s = torch.from_numpy(sel).cuda()
    c = torch.from_numpy(counts).cuda()
    got = xqa.decode_pages(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                           context_lens=d.context_lens, page_select=s, select_counts=c,
                           scale=w.scale, out=out)
    torch.cuda.synchronize()
    return got


def reference(w, sel, counts):
    kp, vp = w.pools()
    return oracle.decode_attention_pages(w.q, kp, vp, w.block_table, w.context_lens, sel, counts,
                                         w.scale)


def log(label, st):
    print(f"[pages] {label}: max_abs={st['max_abs']:.3e} rel_l2={st['rel_l2']:.3e} n={st['n']}",
          flush=True)


@pytest.mark.parametrize("hkv,hq", [(1, 8), (2, 16), (4, 32), (1, 1), (2, 32), (3, 9)])
def test_ragged_messy_selection_vs_oracle(hkv, hq):
    lens = [1, 17, 300, 5000, 0, 33, 2047, 16, 1023, 4100]
    w = make_custom(lens, hkv, hq, [61, hkv, hq], pool_pages=800)
    sel, counts = make_selection(lens, w.max_pages_per_seq, 0.3, [62, hkv, hq], messy=True)
    xqa = handle_for(w)
    d = to_device(w)
    got = run_pages(xqa, w, d, sel, counts).float().cpu().numpy()
    st = assert_parity(got, reference(w, sel, counts), f"ragged hkv={hkv} hq={hq}")
    log(f"ragged hkv={hkv} hq={hq}", st)
    xqa.close()


@pytest.mark.parametrize("items_per_head", [1, 2, 5])
def test_few_work_items_span_sequences(items_per_head):
    # Few items per KV head: items run many segments of the gathered table,
    # and long selections leave states in several items.
    lens = [5000, 17, 0, 2047, 1, 3000, 640, 33]
    w = make_custom(lens, 2, 16, [78, items_per_head], pool_pages=700)
    sel, counts = make_selection(lens, w.max_pages_per_seq, 0.6, [79, items_per_head], messy=True)
    xqa = handle_for(w, max_work_items=2 * items_per_head)
    d = to_device(w)
    got = run_pages(xqa, w, d, sel, counts).float().cpu().numpy()
    st = assert_parity(got, reference(w, sel, counts), f"items/head {items_per_head}")
    log(f"items/head {items_per_head}", st)
    xqa.close()


def test_every_page_in_order_is_decode_bit_for_bit():
    w = make_config(4)
    d = to_device(w)
    xqa = handle_for(w)
    S = w.max_pages_per_seq
    sel = np.tile(np.arange(S, dtype=np.int32), (w.batch, 1))
    counts = np.full(w.batch, S, dtype=np.int32)
    got = run_pages(xqa, w, d, sel, counts)
    ref = xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                     context_lens=d.context_lens, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    xqa.close()


def test_ragged_b16_quarter_of_the_pages_vs_oracle():
    w = make_config(4)
    d = to_device(w)
    xqa = handle_for(w)
    sel, counts = make_selection(w.context_lens, w.max_pages_per_seq, 0.25, [63, 4])
    got = run_pages(xqa, w, d, sel, counts).float().cpu().numpy()
    st = assert_parity(got, reference(w, sel, counts), "ragged b16 quarter")
    log("ragged b16 quarter", st)
    xqa.close()


def test_edge_selections():
    lens = [40, 40, 40, 40, 0, 1, 33, 48, 40]
    w = make_custom(lens, 2, 16, [64], pool_pages=64, max_pages_per_seq=4)
    S = 4
    sel = np.array([[0, 1, 2, -1],     # count 0: nothing selected
                    [0, 1, 2, 3],      # negative count
                    [0, 2, 1, 0],      # count past the stride: clamped to 4; 1 and 0 skipped
                    [3, 5, -2, 9],     # only out-of-range pages
                    [0, 1, 2, 3],      # empty sequence
                    [0, 0, 0, 0],      # one token
                    [2, 2, 2, 2],      # only the partial page holding token 32
                    [2, 1, 0, 3],      # descending: only page 2 kept (a full page)
                    [1, 2, 3, 3]],     # pages 1, 2 (partial); 3 out of range
                   dtype=np.int32)
    counts = np.array([0, -3, 9, 4, 4, 4, 4, 4, 4], dtype=np.int32)
    xqa = handle_for(w, stride=S)
    d = to_device(w)
    got = run_pages(xqa, w, d, sel, counts).float().cpu().numpy()
    ref = reference(w, sel, counts)
    assert_parity(got, ref, "edges")
    for b in (0, 1, 3, 4):
        assert (got[b] == 0).all()
    # One kept token: its V row exactly (softmax weight 1).
    kp, vp = w.pools()
    for b, t in ((5, 0), (6, 32)):
        vrow = oracle.decode_e5m2(vp[w.block_table[b, t // 16], :, t % 16, :])
        for hq in range(16):
            assert np.array_equal(got[b, hq], vrow[hq // 8])
    xqa.close()


def test_pages_left_out_never_matter():
    lens = [700, 129, 4096, 31]
    w = make_custom(lens, 2, 16, [65], pool_pages=400)
    sel, counts = make_selection(lens, w.max_pages_per_seq, 0.4, [66])
    xqa = handle_for(w)
    d = to_device(w)
    before = run_pages(xqa, w, d, sel, counts).clone()
    for b, n in enumerate(lens):
        used = -(-n // 16)
        kept = set(oracle.kept_pages(sel, counts, n, 16, b))
        for p in range(used):
            if p not in kept:
                pg = int(w.block_table[b, p])
                d.k_pages[pg] = 0x7F
                d.v_pages[pg] = 0x7F
    after = run_pages(xqa, w, d, sel, counts)
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))
    xqa.close()


def test_one_kernel_handle():
    # At most 2 pages (32 tokens) per sequence: no sequence is ever split, the
    # split kernel writes every row, zero rows included.
    lens = [32, 0, 17, 5, 31, 0, 16, 1] * 9
    w = make_custom(lens, 4, 32, [67], pool_pages=200, max_pages_per_seq=2)
    sel, counts = make_selection(lens, 2, 0.5, [68], messy=True)
    xqa = handle_for(w, stride=2)
    assert xqa.info["kernels_per_step"] == 1
    d = to_device(w)
    out = torch.full_like(d.q, float("nan"))
    got = run_pages(xqa, w, d, sel, counts, out=out).float().cpu().numpy()
    assert_parity(got, reference(w, sel, counts), "one-kernel")
    xqa.close()


def test_graph_replays_with_changed_selections_equal_eager():
    lens = [3000, 64, 1025, 7000, 0, 513]
    w = make_custom(lens, 4, 32, [69], pool_pages=900)
    d = to_device(w)
    xqa = handle_for(w)
    S = w.max_pages_per_seq
    sels = [make_selection(lens, S, f, [70, i], messy=(i % 2 == 1)) for i, f in
            enumerate([0.1, 0.5, 0.9, 0.3])]
    s_dev = torch.zeros((w.batch, S), dtype=torch.int32, device="cuda")
    c_dev = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    out = torch.empty_like(d.q)
    args = dict(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                context_lens=d.context_lens, page_select=s_dev, select_counts=c_dev, scale=w.scale,
                out=out)
    s_dev.copy_(torch.from_numpy(sels[0][0]))
    c_dev.copy_(torch.from_numpy(sels[0][1]))
    xqa.decode_pages(**args)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xqa.decode_pages(**args)
    for rep in range(8):
        sel, cnt = sels[rep % len(sels)]
        s_dev.copy_(torch.from_numpy(sel))
        c_dev.copy_(torch.from_numpy(cnt))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        replay = out.clone()
        eager = run_pages(xqa, w, d, sel, cnt)
        assert torch.equal(replay.view(torch.int16), eager.view(torch.int16)), rep
        if rep < len(sels):
            assert_parity(replay.float().cpu().numpy(), reference(w, sel, cnt), f"graph {rep}")
    xqa.close()


def test_errors_fail_closed():
    from decode_attention_paged_e5m2_amd import _lib
    lib = _lib.load()
    w = make_custom([100, 50], 1, 8, [71], pool_pages=20)
    d = to_device(w)
    sel, counts = make_selection([100, 50], w.max_pages_per_seq, 0.5, [72])
    s = torch.from_numpy(sel).cuda()
    c = torch.from_numpy(counts).cuda()
    out = torch.empty_like(d.q)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())   # noqa: E731

    def call(xqa, stride, sel_t=s):
        return lib.xqa_decode_pages(xqa._h, P(d.q), P(d.k_pages), P(d.v_pages), P(d.block_table),
                                    P(d.context_lens), P(sel_t), P(c), stride, w.batch,
                                    ctypes.c_float(w.scale), P(out), stream)

    plain = Xqa(max_batch=2, num_q_heads=8, num_kv_heads=1, max_pages_per_seq=w.max_pages_per_seq)
    assert call(plain, w.max_pages_per_seq) == _lib.XQA_ERR_UNSUPPORTED
    xqa = handle_for(w)
    assert call(xqa, w.max_pages_per_seq + 1) == _lib.XQA_ERR_INVALID_ARG
    assert call(xqa, 0) == _lib.XQA_ERR_INVALID_ARG
    assert lib.xqa_decode_pages(xqa._h, P(d.q), P(d.k_pages), P(d.v_pages), P(d.block_table),
                                P(d.context_lens), None, P(c), 1, w.batch, ctypes.c_float(w.scale),
                                P(out), stream) == _lib.XQA_ERR_INVALID_ARG
    assert call(xqa, w.max_pages_per_seq) == _lib.XQA_OK
    torch.cuda.synchronize()
    plain.close()
    xqa.close()
