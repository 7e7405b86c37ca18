"""GPU parity on seeded random mixtures of every input dimension at once:
batch sizes on both sides of 64, ten head shapes (G = 1 to 16), 1 to 8 query
tokens per sequence, E5M2 and E4M3 caches with and without per-tensor scales,
block-table capacities from 128 to 4160 tokens, forced work-item counts,
zero, negative and clamped lengths, and page subsets with messy selection
rows. Every output row is compared against the oracle (the page "[Kernel]
[SM70] Pipeline batched E5M2 XQA decode", sections Purpose and Pending work
and gates: randomized pages, ragged and boundary lengths). The same kind of
mixtures also go through the paths that must agree bit for bit: the fused
append + decode against append then decode, the no-alloc entry point against
a handle, and graph replays against eager calls. A third test takes page
subsets with selection rows longer than the selection kernel's 1,024-entry
tile."""

import numpy as np
import pytest
import torch

import oracle
from tests._helpers import assert_parity, ensure_library
from workloads import make_custom
from workloads.device import to_device

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (1, 8), (2, 4), (4, 8), (8, 2), (3, 5), (1, 16), (2, 16), (6, 1), (4, 3)]


def _selection(rng, lens, cap, cap_pages, batch):
    """Sorted random page subsets of each sequence's used pages, some rows with
    an out-of-order or out-of-range entry inserted, some counts out of range."""
    S = cap_pages
    sel = np.full((batch, S), -1, dtype=np.int32)
    cnt = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        used = (max(0, min(int(lens[b]), cap)) + 15) // 16
        k = int(rng.integers(0, S + 1))
        if used > 0:
            row = list(np.sort(rng.choice(used, size=min(k, used), replace=False)))
        else:
            row = []
        if rng.random() < 0.3 and len(row) < S:
            row.insert(int(rng.integers(0, len(row) + 1)), int(rng.integers(-3, used + 5)))
        row = row[:S]
        sel[b, :len(row)] = row
        cnt[b] = len(row) if rng.random() < 0.9 else int(rng.integers(-2, S + 3))
    return sel, cnt


def test_random_mixtures_against_the_oracle():
    ensure_library()
    from decode_attention_paged_e5m2_amd import Xqa
    rng = np.random.default_rng(20261203)
    for case in range(80):
        batch = int(rng.choice([1, 2, 3, 5, 8, 16, 31, 33, 64, 65, 100, 150]))
        hkv, g = SHAPES[case % len(SHAPES)]
        M = int(rng.choice([m for m in (1, 1, 2, 3, 4, 8) if m <= 16 // g]))
        fmt = "e4m3" if rng.random() < 0.35 else "e5m2"
        if rng.random() < 0.5:
            ks, vs = 1.0, 1.0
        else:
            ks, vs = float(rng.choice([0.25, 0.5, 2.0])), float(rng.choice([0.5, 1.5, 3.0]))
        kind = rng.random(batch)
        cap_pages = int(rng.choice([8, 40, 130, 260]))
        cap = cap_pages * 16
        ctx = np.where(kind < 0.4, rng.integers(1, 80, batch),
                       np.where(kind < 0.85, rng.integers(80, 900, batch),
                                rng.integers(900, 4200, batch)))
        ctx = np.minimum(ctx, cap)
        ctx[rng.random(batch) < 0.08] = 0
        clamp = rng.random(batch) < 0.06
        ctx[clamp] = cap                      # every page of the row is used ...
        w = make_custom(ctx.tolist(), hkv, hkv * g, [777, case], max_pages_per_seq=cap_pages,
                        kv_format=fmt)
        lens = ctx.copy()
        neg = (ctx == 0) & (rng.random(batch) < 0.5)
        lens[neg] = -int(rng.integers(1, 100))
        lens[clamp] = cap + rng.integers(1, 5000, int(clamp.sum()))   # ... and the length clamps
        per_head = int(rng.choice([0, 0, 1, 2, 3, 7, 16, 50]))
        pages = M == 1 and fmt == "e5m2"
        dev = to_device(w)
        dev_lens = torch.from_numpy(lens.astype(np.int32)).to(dev.q.device)
        q = rng.standard_normal((batch, M, hkv * g, 128)).astype(np.float16)
        qq = q if M > 1 else q[:, 0]
        xqa = Xqa(max_batch=batch, num_q_heads=hkv * g, num_kv_heads=hkv,
                  max_pages_per_seq=cap_pages, max_work_items=hkv * per_head, max_query_tokens=M,
                  max_selected_pages=cap_pages if pages else 0)
        tag = (f"case {case} B={batch} hkv={hkv} g={g} M={M} {fmt} k_scale={ks} v_scale={vs} "
               f"cap={cap} per_head={per_head}")
        print(tag, flush=True)
        kp, vp = w.pools()
        out = xqa.decode(q=torch.from_numpy(qq).cuda(), k_pages=dev.k_pages, v_pages=dev.v_pages,
                         block_table=dev.block_table, context_lens=dev_lens, scale=w.scale,
                         kv_format=fmt, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        ref = oracle.decode_attention_fp8(qq, kp, vp, w.block_table, lens, w.scale,
                                          kv_format=fmt, k_scale=ks, v_scale=vs)
        assert_parity(out.float().cpu().numpy(), ref, tag)
        if pages:
            sel, cnt = _selection(rng, lens, cap, cap_pages, batch)
            outp = xqa.decode_pages(q=torch.from_numpy(qq).cuda(), k_pages=dev.k_pages,
                                    v_pages=dev.v_pages, block_table=dev.block_table,
                                    context_lens=dev_lens, page_select=torch.from_numpy(sel).cuda(),
                                    select_counts=torch.from_numpy(cnt).cuda(), scale=w.scale)
            torch.cuda.synchronize()
            refp = oracle.decode_attention_pages(qq, kp, vp, w.block_table, lens, sel, cnt,
                                                 w.scale)
            assert_parity(outp.float().cpu().numpy(), refp, tag + " page subsets")
        xqa.close()
        del dev


def test_random_mixtures_bitwise_paths():
    # The same kind of random mixtures (one query token, E5M2) through the
    # paths that must agree bit for bit: the fused append + decode against
    # the append followed by decode (outputs and pools), xqa_decode_noalloc
    # against a handle, and graph replays against the eager call.
    import ctypes
    lib = ensure_library()
    from decode_attention_paged_e5m2_amd import Xqa
    from decode_attention_paged_e5m2_amd._lib import XqaConfig
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rng = np.random.default_rng(5150)
    for case in range(30):
        batch = int(rng.choice([1, 2, 5, 16, 33, 64, 65, 100]))
        hkv, g = SHAPES[case % len(SHAPES)]
        cap_pages = int(rng.choice([8, 40, 130, 260]))
        cap = cap_pages * 16
        kind = rng.random(batch)
        ctx = np.where(kind < 0.4, rng.integers(1, 80, batch),
                       np.where(kind < 0.85, rng.integers(80, 900, batch),
                                rng.integers(900, 4200, batch)))
        ctx = np.minimum(ctx, cap)
        ctx[rng.random(batch) < 0.08] = 0
        clamp = rng.random(batch) < 0.06
        ctx[clamp] = cap
        w = make_custom(ctx.tolist(), hkv, hkv * g, [991, case], max_pages_per_seq=cap_pages)
        lens = ctx.copy()
        neg = (ctx == 0) & (rng.random(batch) < 0.5)
        lens[neg] = -int(rng.integers(1, 100))
        lens[clamp] = cap + rng.integers(1, 5000, int(clamp.sum()))
        per_head = int(rng.choice([0, 0, 1, 2, 3, 7, 16]))
        tag = f"case {case} B={batch} hkv={hkv} g={g} cap={cap} per_head={per_head}"
        print(tag, flush=True)
        lens_t = torch.from_numpy(lens.astype(np.int32)).cuda()
        xqa = Xqa(max_batch=batch, num_q_heads=hkv * g, num_kv_heads=hkv,
                  max_pages_per_seq=cap_pages, max_work_items=hkv * per_head)
        k_new = torch.from_numpy((rng.standard_normal((batch, hkv, 128)) * 3).astype(np.float16)).cuda()
        v_new = torch.from_numpy(rng.standard_normal((batch, hkv, 128)).astype(np.float16)).cuda()
        sep, fused = to_device(w), to_device(w)
        xqa.append_kv(k_new=k_new, v_new=v_new, block_table=sep.block_table, context_lens=lens_t,
                      k_pages=sep.k_pages, v_pages=sep.v_pages)
        out_sep = xqa.decode(q=sep.q, k_pages=sep.k_pages, v_pages=sep.v_pages,
                             block_table=sep.block_table, context_lens=lens_t, scale=w.scale)
        out_fused = xqa.decode_append(q=fused.q, k_new=k_new, v_new=v_new, k_pages=fused.k_pages,
                                      v_pages=fused.v_pages, block_table=fused.block_table,
                                      context_lens=lens_t, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out_fused.view(torch.int16), out_sep.view(torch.int16)), tag
        assert torch.equal(fused.k_pages, sep.k_pages) and torch.equal(fused.v_pages, sep.v_pages), tag
        kp, vp = w.pools()
        kr, vr = oracle.append_kv(kp, vp, w.block_table, lens, k_new.cpu().numpy(),
                                  v_new.cpu().numpy())
        ref = oracle.decode_attention(w.q, kr, vr, w.block_table, lens, w.scale)
        assert_parity(out_fused.float().cpu().numpy(), ref, tag + " append")
        cfg = XqaConfig(batch, hkv * g, hkv, 128, 16, cap_pages, hkv * per_head, 1, 0)
        out_na = torch.empty_like(out_sep).fill_(float("nan"))
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.xqa_decode_noalloc(ctypes.byref(cfg), p(sep.q), p(sep.k_pages), p(sep.v_pages),
                                    p(sep.block_table), p(lens_t), batch, ctypes.c_float(w.scale),
                                    p(out_na), stream)
        torch.cuda.synchronize()
        assert rc == 0, tag
        assert torch.equal(out_na.view(torch.int16), out_sep.view(torch.int16)), tag + " noalloc"
        out_g = torch.empty_like(out_sep)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            xqa.decode(q=sep.q, k_pages=sep.k_pages, v_pages=sep.v_pages,
                       block_table=sep.block_table, context_lens=lens_t, scale=w.scale, out=out_g)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            xqa.decode(q=sep.q, k_pages=sep.k_pages, v_pages=sep.v_pages,
                       block_table=sep.block_table, context_lens=lens_t, scale=w.scale, out=out_g)
        for r in range(3):
            out_g.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_g.view(torch.int16), out_sep.view(torch.int16)), f"{tag} replay {r}"
        del graph
        xqa.close()


def test_random_page_subsets_over_several_tiles():
    # Page-subset decode with selection rows longer than the selection
    # kernel's 1,024-entry tile (up to 3,000 pages per sequence), selection
    # strides below the handle's capacity, planted out-of-range, repeated and
    # descending entries, and random counts; every row against the oracle,
    # and selecting every page in order bitwise equal to plain decode.
    ensure_library()
    from decode_attention_paged_e5m2_amd import Xqa
    rng = np.random.default_rng(4243)
    for case in range(16):
        hkv, g = SHAPES[case % len(SHAPES)]
        batch = int(rng.choice([1, 2, 3]))
        cap_pages = int(rng.choice([1100, 2100, 3000]))
        cap = cap_pages * 16
        ctx = rng.integers(1, cap + 1, batch)
        ctx[rng.random(batch) < 0.2] = cap
        w = make_custom(ctx.tolist(), hkv, hkv * g, [4243, case], max_pages_per_seq=cap_pages)
        lens = ctx.copy()
        lens[ctx == cap] += rng.integers(0, 3000, int((ctx == cap).sum()))   # clamped lengths
        max_sel = cap_pages if case % 2 == 0 else int(rng.integers(1025, cap_pages + 1))
        S = max_sel if case % 4 < 2 else int(rng.integers(1025, max_sel + 1))
        sel = np.full((batch, S), -1, dtype=np.int32)
        cnt = np.zeros(batch, dtype=np.int32)
        for b in range(batch):
            used = (min(int(lens[b]), cap) + 15) // 16
            row = list(np.sort(rng.choice(used, size=min(int(rng.integers(0, S + 1)), used),
                                          replace=False)))
            for _ in range(3):
                if len(row) < S:
                    row.insert(int(rng.integers(0, len(row) + 1)), int(rng.integers(-3, used + 5)))
            sel[b, :len(row)] = row
            cnt[b] = len(row) if b != 1 else S + 7   # one count past the stride (clamped)
        per_head = int(rng.choice([0, 2, 16]))
        tag = f"case {case} B={batch} hkv={hkv} g={g} cap={cap_pages} S={S} max_sel={max_sel}"
        print(tag, flush=True)
        dev = to_device(w)
        lt = torch.from_numpy(lens.astype(np.int32)).cuda()
        xqa = Xqa(max_batch=batch, num_q_heads=hkv * g, num_kv_heads=hkv,
                  max_pages_per_seq=cap_pages, max_work_items=hkv * per_head,
                  max_selected_pages=max_sel)
        out = xqa.decode_pages(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                               block_table=dev.block_table, context_lens=lt,
                               page_select=torch.from_numpy(sel).cuda(),
                               select_counts=torch.from_numpy(cnt).cuda(), scale=w.scale)
        torch.cuda.synchronize()
        kp, vp = w.pools()
        ref = oracle.decode_attention_pages(w.q, kp, vp, w.block_table, lens, sel, cnt, w.scale)
        assert_parity(out.float().cpu().numpy(), ref, tag)
        if max_sel == cap_pages:
            allp = torch.arange(cap_pages, dtype=torch.int32).repeat(batch, 1).cuda()
            outa = xqa.decode_pages(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                                    block_table=dev.block_table, context_lens=lt, page_select=allp,
                                    select_counts=torch.full((batch,), cap_pages,
                                                             dtype=torch.int32).cuda(),
                                    scale=w.scale)
            outd = xqa.decode(q=dev.q, k_pages=dev.k_pages, v_pages=dev.v_pages,
                              block_table=dev.block_table, context_lens=lt, scale=w.scale)
            torch.cuda.synchronize()
            assert torch.equal(outa.view(torch.int16), outd.view(torch.int16)), tag + " every page"
        xqa.close()
        del dev
