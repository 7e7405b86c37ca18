"""GPU parity of FP8 caches with per-tensor scales (xqa_decode_fp8): E4M3 and
scaled E5M2, single- and multi-token, against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from oracle.e4m3 import E4M3_TABLE
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


def _ref(w, q, k_scale, v_scale, fmt):
    kp, vp = w.pools()
    return oracle.decode_attention_fp8(q, kp, vp, w.block_table, w.context_lens, w.scale,
                                       kv_format=fmt, k_scale=k_scale, v_scale=v_scale)


def _run(w, q=None, k_scale=1.0, v_scale=1.0, fmt="e4m3", max_work_items=0, M=1):
    dev = to_device(w)
    xqa = Xqa(max_batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
              max_pages_per_seq=w.max_pages_per_seq, max_work_items=max_work_items,
              max_query_tokens=M)
    qd = dev.q if q is None else torch.from_numpy(q).to(dev.q.device)
    out = xqa.decode(q=qd, k_pages=dev.k_pages, v_pages=dev.v_pages, block_table=dev.block_table,
                     context_lens=dev.context_lens, scale=w.scale, kv_format=fmt,
                     k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def test_widen_e4m3_all_256_codes_bit_exact():
    from decode_attention_paged_e5m2_amd import debug_widen_e4m3
    for n in (256, 1001):
        codes = np.arange(n, dtype=np.int64) % 256
        bits, vals = debug_widen_e4m3(torch.from_numpy(codes.astype(np.uint8)).cuda())
        bits = bits.cpu().numpy().view(np.uint16)
        vals = vals.cpu().numpy()
        want = E4M3_TABLE[codes]
        nan = np.isnan(want)
        # Every E4M3 value is a binary16 value: the bits are the exact pattern.
        assert np.array_equal(bits[~nan], want[~nan].astype(np.float16).view(np.uint16))
        assert np.isnan(vals[nan]).all() and np.array_equal(vals[~nan], want[~nan])


@pytest.mark.parametrize("hkv,hq,k_scale,v_scale", [
    (4, 32, 1.0, 1.0), (4, 32, 0.5, 2.0), (2, 16, 0.03125, 0.7), (1, 8, 3.0, 0.001), (8, 8, 1.7, 5.0),
])
def test_e4m3_sweep(hkv, hq, k_scale, v_scale):
    lens = [1, 15, 16, 17, 31, 32, 33, 300, 2049, 0, 5000]
    w = make_custom(lens, hkv, hq, [71, hkv, hq], pool_pages=800, kv_format="e4m3")
    out = _run(w, k_scale=k_scale, v_scale=v_scale)
    assert_parity(out, _ref(w, w.q, k_scale, v_scale, "e4m3"),
                  f"e4m3 hkv={hkv} hq={hq} ks={k_scale} vs={v_scale}")


def test_e4m3_with_outliers_saturating_at_448():
    # 1% of the values x1000: they saturate at 448 in the cache.
    w = make_custom([700, 64, 3000], 4, 32, [72, 0], pool_pages=300, kv_format="e4m3",
                    outlier_frac=0.01)
    out = _run(w, k_scale=0.25, v_scale=1.5)
    assert_parity(out, _ref(w, w.q, 0.25, 1.5, "e4m3"), "e4m3 outliers")


def test_e4m3_two_query_tokens_and_item_boundaries():
    lens = [33, 64, 65, 255, 256, 1000, 2, 1]
    w = make_custom(lens, 4, 32, [73, 0], pool_pages=200, kv_format="e4m3")
    q = np.random.default_rng(74).standard_normal((w.batch, 2, 32, 128)).astype(np.float16)
    for per_head in (0, 3):
        out = _run(w, q=q, k_scale=0.8, v_scale=1.25, max_work_items=4 * per_head, M=2)
        assert_parity(out, _ref(w, q, 0.8, 1.25, "e4m3"), f"e4m3 M=2 per_head={per_head}")


def test_e5m2_with_scales():
    w = make_custom([1, 100, 2049, 33, 0], 4, 32, [75, 0], pool_pages=300)
    out = _run(w, k_scale=0.125, v_scale=3.0, fmt="e5m2")
    assert_parity(out, _ref(w, w.q, 0.125, 3.0, "e5m2"), "e5m2 scaled")


def test_e4m3_full_size_ragged_b16():
    w = make_config(4, kv_format="e4m3")
    out = _run(w, k_scale=0.5, v_scale=2.0)
    assert_parity(out, _ref(w, w.q, 0.5, 2.0, "e4m3"), "cfg4 e4m3")


def test_e4m3_graph_replays_equal_eager():
    w = make_custom([900, 17, 4100], 2, 16, [76, 0], pool_pages=400, kv_format="e4m3")
    dev = to_device(w)
    xqa = Xqa(max_batch=3, num_q_heads=16, num_kv_heads=2, max_pages_per_seq=w.max_pages_per_seq)
    out = torch.empty_like(dev.q)

    def step():
        xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages, block_table=dev.block_table,
                   context_lens=dev.context_lens, scale=w.scale, out=out, kv_format="e4m3",
                   k_scale=0.5, v_scale=2.0)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(6):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
    assert_parity(eager.float().cpu().numpy(), _ref(w, w.q, 0.5, 2.0, "e4m3"), "e4m3 graph")
