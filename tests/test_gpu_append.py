"""GPU parity of the KV append (xqa_append_kv) against the oracle, through the C ABI.

Byte work, so the bar is bit-exact: the whole K and V pools after the call
must equal oracle.append_kv's, which also proves that nothing outside the
target slots was written.
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


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


def _random_pools(rng, num_pages, hkv):
    shape = (num_pages, hkv, 16, 128)
    return (rng.integers(0, 256, size=shape, dtype=np.uint8),
            rng.integers(0, 256, size=shape, dtype=np.uint8))


def _run_append(xqa, k, v, bt, lens, k_new, v_new):
    kd, vd = _dev(k), _dev(v)
    xqa.append_kv(k_new=_dev(k_new), v_new=_dev(v_new), block_table=_dev(bt),
                  context_lens=_dev(lens.astype(np.int32)), k_pages=kd, v_pages=vd)
    torch.cuda.synchronize()
    return kd.cpu().numpy(), vd.cpu().numpy()


def test_append_every_fp16_pattern_bit_exact():
    # 64 sequences x 4 KV heads x 128 values x (K, V) = 65536: every binary16
    # bit pattern is encoded exactly once (subnormals, midpoints, values past
    # 57344, +-inf, NaNs, -0).
    rng = np.random.default_rng(21)
    B, hkv, max_pages = 64, 4, 3
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng.shuffle(bits)
    k_new = bits[:32768].view(np.float16).reshape(B, hkv, 128)
    v_new = bits[32768:].view(np.float16).reshape(B, hkv, 128)
    k, v = _random_pools(rng, B * max_pages, hkv)
    bt = rng.permutation(B * max_pages).reshape(B, max_pages).astype(np.int32)
    lens = rng.integers(1, max_pages * 16 + 1, size=B)
    xqa = Xqa(max_batch=B, num_q_heads=hkv * 8, num_kv_heads=hkv, max_pages_per_seq=max_pages)
    kg, vg = _run_append(xqa, k, v, bt, lens, k_new, v_new)
    kr, vr = oracle.append_kv(k, v, bt, lens, k_new, v_new)
    assert np.array_equal(kg, kr), f"K pool differs at {np.argwhere(kg != kr)[:5]}"
    assert np.array_equal(vg, vr), f"V pool differs at {np.argwhere(vg != vr)[:5]}"


def test_append_edge_lengths_bit_exact():
    # Slot 0 of a page, slot 15, the last slot of the table, and lengths that
    # must not write (0, negative, one past the capacity).
    rng = np.random.default_rng(22)
    hkv, max_pages = 2, 4
    lens = np.array([1, 16, 17, 32, 33, 64, 0, -5, 65, 40, 2], dtype=np.int64)
    B = lens.size
    k, v = _random_pools(rng, B * max_pages + 3, hkv)
    bt = rng.permutation(B * max_pages + 3)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    k_new = (rng.standard_normal((B, hkv, 128)) * 100).astype(np.float16)
    v_new = (rng.standard_normal((B, hkv, 128)) * 1e-5).astype(np.float16)
    xqa = Xqa(max_batch=B, num_q_heads=16, num_kv_heads=hkv, max_pages_per_seq=max_pages)
    kg, vg = _run_append(xqa, k, v, bt, lens, k_new, v_new)
    kr, vr = oracle.append_kv(k, v, bt, lens, k_new, v_new)
    assert np.array_equal(kg, kr)
    assert np.array_equal(vg, vr)
    changed = (kg != k).any(axis=(1, 2, 3)).sum() + (vg != v).any(axis=(1, 2, 3)).sum()
    assert changed > 0


def test_append_then_decode_matches_the_oracle():
    # Decode right after the append, on the same stream, sees the new token.
    lens_after = [1, 17, 300, 4096, 33, 0, 5000, 16]
    w = make_custom(lens_after, 4, 32, [23, 0], pool_pages=800)
    dev = to_device(w)
    rng = np.random.default_rng(24)
    k_new = rng.standard_normal((w.batch, 4, 128)).astype(np.float16)
    v_new = (rng.standard_normal((w.batch, 4, 128)) * 2).astype(np.float16)
    xqa = Xqa(max_batch=w.batch, num_q_heads=32, num_kv_heads=4,
              max_pages_per_seq=w.max_pages_per_seq)
    xqa.append_kv(k_new=_dev(k_new), v_new=_dev(v_new), block_table=dev.block_table,
                  context_lens=dev.context_lens, k_pages=dev.k_pages, v_pages=dev.v_pages)
    out = xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                     block_table=dev.block_table, context_lens=dev.context_lens, scale=w.scale)
    torch.cuda.synchronize()
    kp, vp = w.pools()
    kr, vr = oracle.append_kv(kp, vp, w.block_table, w.context_lens, k_new, v_new)
    # The device pools hold poison in unused slots; compare only referenced pages.
    used = np.unique(w.block_table[w.block_table != kp.shape[0] - 1])
    assert np.array_equal(dev.k_pages.cpu().numpy()[used], kr[used])
    assert np.array_equal(dev.v_pages.cpu().numpy()[used], vr[used])
    ref = oracle.decode_attention(w.q, kr, vr, w.block_table, w.context_lens, w.scale)
    assert_parity(out.float().cpu().numpy(), ref, "append then decode")


def test_append_and_decode_in_one_graph():
    # One captured graph holding append + decode, replayed with new token rows
    # and new lengths each time; every replay equals the eager calls.
    lens0 = np.array([40, 7, 300, 1], dtype=np.int64)
    w = make_custom((lens0 + 8).tolist(), 2, 16, [25, 0], pool_pages=200)
    rng = np.random.default_rng(26)
    xqa = Xqa(max_batch=w.batch, num_q_heads=16, num_kv_heads=2,
              max_pages_per_seq=w.max_pages_per_seq)
    dev = to_device(w)
    k_new = torch.empty((w.batch, 2, 128), dtype=torch.float16, device="cuda:0")
    v_new = torch.empty_like(k_new)
    lens = torch.empty(w.batch, dtype=torch.int32, device="cuda:0")
    out = torch.empty_like(dev.q)
    kp0, vp0 = dev.k_pages.clone(), dev.v_pages.clone()

    def step():
        xqa.append_kv(k_new=k_new, v_new=v_new, block_table=dev.block_table, context_lens=lens,
                      k_pages=dev.k_pages, v_pages=dev.v_pages)
        xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                   block_table=dev.block_table, context_lens=lens, scale=w.scale, out=out)

    def set_inputs(i):
        k_new.copy_(torch.from_numpy(rng.standard_normal((w.batch, 2, 128)).astype(np.float16)))
        v_new.copy_(torch.from_numpy(rng.standard_normal((w.batch, 2, 128)).astype(np.float16)))
        lens.copy_(torch.from_numpy((lens0 + 1 + (i % 8)).astype(np.int32)))

    stream = torch.cuda.Stream()
    set_inputs(0)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step()                      # warm up outside capture
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for i in range(12):
        dev.k_pages.copy_(kp0)
        dev.v_pages.copy_(vp0)
        set_inputs(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_out, got_k, got_v = out.clone(), dev.k_pages.clone(), dev.v_pages.clone()
        dev.k_pages.copy_(kp0)
        dev.v_pages.copy_(vp0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got_k, dev.k_pages) and torch.equal(got_v, dev.v_pages), f"replay {i}"
        assert torch.equal(got_out.view(torch.int16), out.view(torch.int16)), f"replay {i}"


@pytest.mark.parametrize("per_head", [0, 1, 3])
def test_fused_append_decode_is_bitwise_append_then_decode(per_head):
    # xqa_decode_append == xqa_append_kv; xqa_decode, bit for bit (output and
    # pools): slot 0, slot 15, block edges, the table's capacity, a length
    # past it (clamped, nothing written), empty and negative lengths, and long
    # sequences whose last block falls in later 32-block chunks of a wave.
    cap_pages = 330
    lens = [1, 16, 17, 32, 33, 64, 0, -3, cap_pages * 16 + 9, 300, 5000, cap_pages * 16]
    alloc = [max(0, min(n, cap_pages * 16)) for n in lens]
    w = make_custom(alloc, 4, 32, [27, per_head], pool_pages=1400, max_pages_per_seq=cap_pages)
    rng = np.random.default_rng(28 + per_head)
    k_new = _dev((rng.standard_normal((w.batch, 4, 128)) * 3).astype(np.float16))
    v_new = _dev(rng.standard_normal((w.batch, 4, 128)).astype(np.float16))
    lens_t = _dev(np.asarray(lens, dtype=np.int32))
    xqa = Xqa(max_batch=w.batch, num_q_heads=32, num_kv_heads=4, max_pages_per_seq=cap_pages,
              max_work_items=4 * per_head)
    sep, fused = to_device(w), to_device(w)
    xqa.append_kv(k_new=k_new, v_new=v_new, block_table=sep.block_table, context_lens=lens_t,
                  k_pages=sep.k_pages, v_pages=sep.v_pages)
    out_sep = xqa.decode(q=sep.q, k_pages=sep.k_pages, v_pages=sep.v_pages,
                         block_table=sep.block_table, context_lens=lens_t, scale=w.scale)
    out_fused = xqa.decode_append(q=fused.q, k_new=k_new, v_new=v_new, k_pages=fused.k_pages,
                                  v_pages=fused.v_pages, block_table=fused.block_table,
                                  context_lens=lens_t, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out_fused.view(torch.int16), out_sep.view(torch.int16))
    assert torch.equal(fused.k_pages, sep.k_pages) and torch.equal(fused.v_pages, sep.v_pages)
    kp, vp = w.pools()
    kr, vr = oracle.append_kv(kp, vp, w.block_table, np.asarray(lens), k_new.cpu().numpy(),
                              v_new.cpu().numpy())
    ref = oracle.decode_attention(w.q, kr, vr, w.block_table, np.asarray(lens), w.scale)
    assert_parity(out_fused.float().cpu().numpy(), ref, f"fused append per_head={per_head}")


def test_fused_append_decode_in_a_graph():
    lens0 = np.array([40, 7, 300, 1, 1023], dtype=np.int64)
    w = make_custom((lens0 + 8).tolist(), 4, 32, [29, 0], pool_pages=200)
    rng = np.random.default_rng(30)
    xqa = Xqa(max_batch=w.batch, num_q_heads=32, num_kv_heads=4,
              max_pages_per_seq=w.max_pages_per_seq)
    a, b = to_device(w), to_device(w)
    k_new = torch.empty((w.batch, 4, 128), dtype=torch.float16, device="cuda:0")
    v_new = torch.empty_like(k_new)
    lens = torch.empty(w.batch, dtype=torch.int32, device="cuda:0")
    out_a = torch.empty_like(a.q)
    out_b = torch.empty_like(b.q)

    def fused():
        xqa.decode_append(q=a.q, k_new=k_new, v_new=v_new, k_pages=a.k_pages, v_pages=a.v_pages,
                          block_table=a.block_table, context_lens=lens, scale=w.scale, out=out_a)

    torch.cuda.synchronize()
    lens.copy_(torch.from_numpy((lens0 + 1).astype(np.int32)))
    fused()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fused()
    for i in range(10):
        k_new.copy_(torch.from_numpy(rng.standard_normal((w.batch, 4, 128)).astype(np.float16)))
        v_new.copy_(torch.from_numpy(rng.standard_normal((w.batch, 4, 128)).astype(np.float16)))
        lens.copy_(torch.from_numpy((lens0 + 1 + (i % 8)).astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        xqa.append_kv(k_new=k_new, v_new=v_new, block_table=b.block_table, context_lens=lens,
                      k_pages=b.k_pages, v_pages=b.v_pages)
        xqa.decode(q=b.q, k_pages=b.k_pages, v_pages=b.v_pages, block_table=b.block_table,
                   context_lens=lens, scale=w.scale, out=out_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"replay {i}"
        assert torch.equal(a.k_pages, b.k_pages) and torch.equal(a.v_pages, b.v_pages), f"replay {i}"
