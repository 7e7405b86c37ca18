"""xqa_decode_noalloc through the C ABI: the handle-free decode whose split
states live in the library's fixed device array. Its
output must equal xqa_decode on a handle made from the same configuration,
bit for bit, on consecutive calls of different sizes; sizes past the fixed
array are rejected before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests._helpers import assert_parity, ensure_library
from workloads import make_custom
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    return ensure_library()


def _cfg(max_batch, hq, hkv, pages, max_work_items=0):
    from decode_attention_paged_e5m2_amd._lib import XqaConfig
    return XqaConfig(max_batch, hq, hkv, 128, 16, pages, max_work_items, 1, 0)


def _noalloc(lib, cfg, d, batch, out):
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.xqa_decode_noalloc(ctypes.byref(cfg), p(d.q), p(d.k_pages), p(d.v_pages),
                                  p(d.block_table), p(d.context_lens), batch,
                                  ctypes.c_float(d.scale), p(out), stream)


def test_noalloc_equals_handle_decode_on_consecutive_calls(lib):
    from decode_attention_paged_e5m2_amd import Xqa
    pages = 1024
    cfg = _cfg(16, 32, 4, pages)
    xqa = Xqa(max_batch=16, num_q_heads=32, num_kv_heads=4, max_pages_per_seq=pages)
    rng = np.random.default_rng(404)
    big = make_custom(rng.integers(1, 16 * pages, size=16).tolist(), 4, 32, [405, 0],
                      max_pages_per_seq=pages)
    small = make_custom([0, 3000, 17, 9000, 1], 4, 32, [405, 1], max_pages_per_seq=pages)
    for w in (big, small):   # the second call is smaller: fewer sequences, other lengths
        d = to_device(w)
        out = torch.full_like(d.q, float("nan"))
        assert _noalloc(lib, cfg, d, w.batch, out) == 0, lib.xqa_last_error()
        ref = xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                         context_lens=d.context_lens, scale=w.scale,
                         out=torch.full_like(d.q, float("nan")))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        kp, vp = w.pools()
        want = oracle.decode_attention(w.q, kp, vp, w.block_table, w.context_lens, w.scale)
        assert_parity(out.float().cpu().numpy(), want, f"noalloc batch {w.batch}")
    xqa.close()


def test_noalloc_graph_replay_matches_eager(lib):
    pages = 256
    cfg = _cfg(4, 16, 2, pages)
    w = make_custom([4000, 1, 2500, 0], 2, 16, [406, 0], max_pages_per_seq=pages)
    d = to_device(w)
    eager = torch.empty_like(d.q)
    assert _noalloc(lib, cfg, d, w.batch, eager) == 0
    torch.cuda.synchronize()
    out = torch.empty_like(d.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert _noalloc(lib, cfg, d, w.batch, out) == 0
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_noalloc_rejects_steps_past_the_fixed_array(lib):
    # 2048 items per KV head of 16 query rows: 2 * 8192 records of 2080 floats,
    # far past 16 MiB; rejected before any launch.
    cfg = _cfg(4, 64, 4, 64, max_work_items=4 * 2048)
    w = make_custom([10, 20, 30, 40], 4, 64, [407, 0], max_pages_per_seq=64)
    d = to_device(w)
    out = torch.full_like(d.q, float("nan"))
    assert _noalloc(lib, cfg, d, w.batch, out) == 2
    assert b"16 MiB" in lib.xqa_last_error()
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    # batch past cfg's max_batch
    assert _noalloc(lib, _cfg(2, 64, 4, 64), d, 4, out) == 1
