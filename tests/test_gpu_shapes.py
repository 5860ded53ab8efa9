"""GPU parity on shapes outside the five measured workloads, so that every compiled kernel
variant runs against the oracle: bf16 with head_dim 64, block sizes 32 and 64, a single query
head per KV head (G = 1, the stored-score SnapKV pass) and eight (G = 8, the largest verify
tile of 32 query rows), SnapKV row-tile counts 1, 4 and 6, the fp32 path at head_dim 128, and
verify row counts 17, 20 (head_dim 64) and 24 (the last 16-row tile folded) and 25 (not).

Each workload is ragged or shuffled and spans several blocks, splits and a partial last block.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oatt
import oracle.snapkv as osnap
from oracle.kvcache import append_rows, compact_rows
from oracle.topk import topk_draft_attention
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate, to_numpy
from kv_sparse_speculative_amd.workloads import Workload

from _helpers import ATTN_RTOL, host, lse_err, row_rel_err

pytestmark = pytest.mark.gpu

#        name               dtype  B  Hq Hkv  D   prompt       gamma streaming  snapkv (budget, w, pool)
SHAPES = [
    Workload("bf16_d64_g4", "bf16", 3, 16, 4, 64, (600, 1100), 3, (4, 60), (96, 16, 7), 1000,
             block_size=16, shuffled_blocks=True, planted_frac=0.02, seed=2001),
    Workload("bf16_g8_bs32", "bf16", 2, 32, 4, 128, (700, 1200), 3, (8, 120), (140, 12, 5), 1000,
             block_size=32, shuffled_blocks=True, planted_frac=0.02, seed=2002),
    Workload("bf16_g1_bs64", "bf16", 3, 4, 4, 128, (500, 900), 7, (16, 48), (80, 16, 3), 1000,
             block_size=64, shuffled_blocks=True, seed=2003),
    Workload("bf16_d64_g2_bs32", "bf16", 4, 8, 4, 64, (300, 800), 5, (4, 28), (100, 24, 9), 1000,
             block_size=32, seed=2004),
    Workload("f32_d128_g5", "f32", 2, 10, 2, 128, (300, 500), 2, (4, 60), (72, 8, 7), 1000,
             seed=2005),
    # verify row counts at the folded-last-tile boundaries: 17 and 24 rows (head_dim 128), 20
    # rows at head_dim 64, and 25 rows (two tiles, not folded)
    Workload("bf16_r17_g1", "bf16", 2, 4, 4, 128, (400, 700), 16, (4, 28), (64, 8, 5), 1000,
             block_size=16, shuffled_blocks=True, seed=2006),
    Workload("bf16_r24_g8", "bf16", 2, 16, 2, 128, (500, 900), 2, (8, 56), (96, 8, 7), 1000,
             block_size=32, seed=2007),
    Workload("bf16_d64_r20_g4", "bf16", 3, 16, 4, 64, (300, 1000), 4, (4, 60), (80, 16, 7), 1000,
             block_size=16, shuffled_blocks=True, seed=2008),
    Workload("bf16_r25_g5", "bf16", 2, 10, 2, 128, (600, 800), 4, (4, 28), (64, 8, 3), 1000,
             block_size=64, seed=2009),
]
IDS = [w.name for w in SHAPES]


@pytest.fixture(scope="module", params=SHAPES, ids=IDS)
def ns(request):
    torch.manual_seed(0)
    wl = request.param
    print(f"\nshape {wl.name}", flush=True)
    out = generate(wl, device="cuda", parts=("attn",))
    torch.cuda.synchronize()
    return out


def _kv(ns, lens, max_len):
    return kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, lens, max_len)


def test_verify_and_decode(ns):
    wl = ns.workload
    P = ns.prompt_lens_np
    scale = 1 / math.sqrt(wl.head_dim)
    qh, kh, vh = host(ns.q_verify), host(ns.k_cache), host(ns.v_cache)
    out, lse = kvss.verify_attn_full(_kv(ns, ns.kv_lens_verify, int(P.max()) + ns.T), ns.q_verify)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.verify_attention(qh, kh, vh, ns.block_table_np, P + ns.T, scale)
    err = row_rel_err(host(out), ref)
    print(f"verify {wl.name}: max row rel err {err:.3e}")
    assert err <= ATTN_RTOL
    assert lse_err(host(lse), ref_lse) <= 1e-4
    # T = 1 over the draft lengths is a plain decode
    q1 = ns.q_draft.unsqueeze(2).contiguous()
    out, lse = kvss.verify_attn_full(_kv(ns, ns.kv_lens_draft, int(P.max()) + 1), q1)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.decode_attention(host(ns.q_draft), kh, vh, ns.block_table_np, P + 1, scale)
    assert row_rel_err(host(out)[:, :, 0], ref) <= ATTN_RTOL
    assert lse_err(host(lse)[:, :, 0], ref_lse) <= 1e-4


def test_snapkv_select_and_drafts(ns):
    wl = ns.workload
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    L = P + 1
    scale = 1 / math.sqrt(wl.head_dim)
    sel, cnt, scores = kvss.snapkv_select(_kv(ns, ns.prompt_lens, int(P.max())), ns.q_obs, w,
                                          pool, budget, want_scores=True)
    torch.cuda.synchronize()
    kh, vh = host(ns.k_cache), host(ns.v_cache)
    ref_c = osnap.snapkv_scores(host(ns.q_obs), kh, ns.block_table_np, P, w, scale)
    g_sel, g_cnt, g_c = host(sel), host(cnt), host(scores)
    for b in range(ns.batch):
        n = max(int(P[b]) - w, 0)
        np.testing.assert_allclose(g_c[b, :, :n], ref_c[b, :, :n], rtol=1e-4, atol=1e-7)
    o_sel, o_cnt = osnap.select_from_scores(g_c.astype(np.float64), P, w, pool, budget)
    np.testing.assert_array_equal(g_sel, o_sel)
    np.testing.assert_array_equal(g_cnt, o_cnt)
    r_sel, r_cnt = osnap.select_from_scores(ref_c, P, w, pool, budget)
    np.testing.assert_array_equal(g_cnt, r_cnt)
    for b in range(ns.batch):
        n = max(int(P[b]) - w, 0)
        for g in range(wl.num_kv_heads):
            diff = set(g_sel[b, g][g_sel[b, g] >= 0].tolist()) ^ set(r_sel[b, g][r_sel[b, g] >= 0].tolist())
            if diff:
                pooled = osnap.max_pool(ref_c[b, g, :n], pool)
                tau = np.sort(pooled)[::-1][budget - w - 1]
                assert all(abs(pooled[j] - tau) <= 1e-5 * tau for j in diff), (b, g)

    kvd = _kv(ns, ns.kv_lens_draft, int(L.max()))
    qh = host(ns.q_draft)
    tail = (ns.prompt_lens - w).contiguous()
    out, lse = kvss.draft_attn_sparse(kvd, ns.q_draft, sel, cnt, tail, w + 1)
    sink, window = wl.streaming
    s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(ns.kv_lens_draft, wl.num_kv_heads, sink, window)
    s_out, s_lse = kvss.draft_attn_sparse(kvd, ns.q_draft, s_idx, s_cnt, s_tail, window)
    torch.cuda.synchronize()
    for label, o, l, si, sc, tl in (("snapkv", out, lse, sel, cnt, tail),
                                    ("streaming", s_out, s_lse, s_idx, s_cnt, s_tail)):
        ref, ref_lse = oatt.draft_attention(qh, kh, vh, ns.block_table_np, L, host(si), host(sc),
                                            host(tl), scale)
        err = row_rel_err(host(o), ref)
        print(f"draft {wl.name} {label}: max row rel err {err:.3e}")
        assert err <= ATTN_RTOL, label
        assert lse_err(host(l), ref_lse) <= 1e-4, label


def test_dynamic_topk_draft(ns):
    wl = ns.workload
    L = ns.prompt_lens_np + 1
    k = wl.snapkv[0] - 1
    kv = _kv(ns, ns.kv_lens_draft, int(L.max()))
    sel = torch.empty((ns.batch, wl.num_kv_heads, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(ns.batch, dtype=torch.int32, device="cuda")
    out, lse = kvss.draft_attn_topk(kv, ns.q_draft, k, sel_idx=sel, sel_count=cnt)
    q_obs = ns.q_draft.unsqueeze(2).contiguous()
    s_sel, s_cnt, scores = kvss.snapkv_select(kv, q_obs, 1, 1, k + 1, want_scores=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sel), host(s_sel))
    np.testing.assert_array_equal(host(cnt), host(s_cnt))
    o_sel, o_cnt = osnap.select_from_scores(host(scores).astype(np.float64), L, 1, 1, k + 1)
    np.testing.assert_array_equal(host(sel), o_sel)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    # the attention over the kept set, against the oracle's attention over that same set
    scale = 1 / math.sqrt(wl.head_dim)
    kh, vh = host(ns.k_cache), host(ns.v_cache)
    tail = (ns.prompt_lens_np).astype(np.int32)
    ref, ref_lse = oatt.draft_attention(host(ns.q_draft), kh, vh, ns.block_table_np, L, host(sel),
                                        host(cnt), tail, scale)
    err = row_rel_err(host(out), ref)
    print(f"dynamic top-k {wl.name}: max row rel err {err:.3e}")
    assert err <= ATTN_RTOL
    assert lse_err(host(lse), ref_lse) <= 1e-4
    # and the oracle's own set agrees except at near-ties of the k-th score
    _, _, r_sel, r_cnt = topk_draft_attention(host(ns.q_draft), kh, vh, ns.block_table_np, L, k, scale)
    np.testing.assert_array_equal(host(cnt), r_cnt)


def test_append_and_compact_cache(ns):
    wl = ns.workload
    P = ns.prompt_lens_np
    L = P + 1
    B, Hkv, D, bs = ns.batch, wl.num_kv_heads, wl.head_dim, wl.block_size
    budget, w, _ = wl.snapkv
    k = budget - w
    rng = np.random.default_rng(wl.seed + 9)
    tail = np.maximum(P - w, 0).astype(np.int32)
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = min(k, int(tail[b]))
        cnt[b] = n
        for g in range(Hkv):
            sel[b, g, :n] = np.sort(rng.choice(int(tail[b]), size=n, replace=False))
    src = _kv(ns, ns.kv_lens_draft, int(L.max()))
    cap = k + w + 1
    cb = (cap + bs - 1) // bs
    dst_table = rng.permutation(B * cb).astype(np.int32).reshape(B, cb)
    dk = torch.zeros((B * cb, Hkv, bs, D), dtype=ns.k_cache.dtype, device="cuda")
    dv = torch.zeros_like(dk)
    dst = kvss.PagedKV(dk, dv, torch.from_numpy(dst_table).cuda(),
                       torch.zeros(B, dtype=torch.int32, device="cuda"), cap)
    t_sel, t_cnt, t_tail = (torch.from_numpy(x).cuda() for x in (sel, cnt, tail))
    lens = kvss.kvss_draft_cache_build(src, t_sel, t_cnt, t_tail, w + 1, dst)
    torch.cuda.synchronize()
    kh, vh = host(ns.k_cache), host(ns.v_cache)
    rk, r_lens = compact_rows(kh, ns.block_table_np, L, sel, cnt, tail, w + 1)
    rv, _ = compact_rows(vh, ns.block_table_np, L, sel, cnt, tail, w + 1)
    np.testing.assert_array_equal(host(lens), r_lens)
    gk, gv = host(dk), host(dv)
    for b in range(B):
        j = np.arange(int(r_lens[b]))
        blk = dst_table[b, j // bs]
        np.testing.assert_array_equal(gk[blk, :, j % bs].transpose(1, 0, 2), rk[b])
        np.testing.assert_array_equal(gv[blk, :, j % bs].transpose(1, 0, 2), rv[b])
    # a decode over the compact cache attends exactly the sparse draft's set
    out, _ = kvss.verify_attn_full(dst.with_lens(lens, cap), ns.q_draft.unsqueeze(2).contiguous())
    torch.cuda.synchronize()
    ref, _ = oatt.draft_attention(host(ns.q_draft), kh, vh, ns.block_table_np, L, sel, cnt, tail,
                                  1 / math.sqrt(D))
    assert row_rel_err(host(out)[:, :, 0], ref) <= ATTN_RTOL

    # append the gamma + 1 verify rows of every sequence at positions P .. P + gamma (new values),
    # on a copy of the cache
    k2, v2 = ns.k_cache.clone(), ns.v_cache.clone()
    gen = torch.Generator().manual_seed(wl.seed)
    kn = torch.randn((B, Hkv, ns.T, D), generator=gen).to(ns.k_cache.dtype).cuda()
    vn = torch.randn((B, Hkv, ns.T, D), generator=gen).to(ns.k_cache.dtype).cuda()
    kva = kvss.PagedKV(k2, v2, ns.block_table, ns.prompt_lens, int(P.max()))
    kvss.kvss_kv_append(kva, kn, vn, ns.prompt_lens)
    torch.cuda.synchronize()
    ref_k, ref_v = append_rows(kh, vh, ns.block_table_np, to_numpy(kn), to_numpy(vn), P.astype(np.int32))
    np.testing.assert_array_equal(host(k2), ref_k)
    np.testing.assert_array_equal(host(v2), ref_v)
