"""Parity at the workloads' full sizes, in the launch configurations bench.py times.

Every call runs on the whole batch exactly as in the benchmark (same shapes, hence the same
split plans); the oracle checks sampled (sequence, KV head) pairs -- first, last and a middle
one -- on host copies of just those sequences' cache blocks, and sampled sequences for
acceptance.
"""

import math

import numpy as np
import pytest
import torch

import oracle.accept as oacc
import oracle.attention as oatt
import oracle.snapkv as osnap
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import ATTN_RTOL, host, lse_err, row_rel_err, subcache

pytestmark = pytest.mark.gpu

FULL = ["llama8b_ctx8k", "llama8b_ctx32k", "llama8b_ctx100k", "qwen32b_ragged"]


def _pairs(B, Hkv):
    return sorted({(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2)})


@pytest.fixture(scope="module", params=FULL)
def full(request):
    wl = WORKLOADS[request.param]
    ns = generate(wl, device="cuda")
    torch.cuda.synchronize()
    yield ns
    del ns
    torch.cuda.empty_cache()


def _sub(ns, b, tensor):
    return host(tensor[b:b + 1])


def test_fullsize_verify(full):
    ns, wl = full, full.workload
    P = ns.prompt_lens_np
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_verify, int(P.max()) + ns.T)
    out, lse = kvss.verify_attn_full(kv, ns.q_verify)
    torch.cuda.synchronize()
    worst = 0.0
    for b, g in _pairs(ns.batch, wl.num_kv_heads):
        k, v, table = subcache(ns, [b])
        ref, ref_lse = oatt.verify_attention(_sub(ns, b, ns.q_verify), k, v, table, P[b:b + 1] + ns.T,
                                             1 / math.sqrt(wl.head_dim), pairs=[(0, g)])
        G = wl.group
        hs = slice(g * G, (g + 1) * G)
        err = row_rel_err(host(out[b, hs]), ref[0, hs])
        worst = max(worst, err)
        assert lse_err(host(lse[b, hs]), ref_lse[0, hs]) <= 1e-4
    print(f"fullsize verify {wl.name}: worst sampled row rel err {worst:.3e}")
    assert worst <= ATTN_RTOL
    assert torch.isfinite(out).all()


def test_fullsize_snapkv_and_draft(full):
    ns, wl = full, full.workload
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    scale = 1 / math.sqrt(wl.head_dim)
    kvp = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, int(P.max()))
    sel, cnt, sc = kvss.snapkv_select(kvp, ns.q_obs, w, pool, budget, want_scores=True)
    kvd = kvp.with_lens(ns.kv_lens_draft, int(P.max()) + 1)
    tail = (ns.prompt_lens - w).contiguous()
    d_out, d_lse = kvss.draft_attn_sparse(kvd, ns.q_draft, sel, cnt, tail, w + 1)
    torch.cuda.synchronize()
    g_sel, g_cnt = host(sel), host(cnt)
    np.testing.assert_array_equal(g_cnt, np.minimum(budget - w, P - w))
    for b, g in _pairs(ns.batch, wl.num_kv_heads):
        k, v, table = subcache(ns, [b])
        n = int(P[b]) - w
        ref_c = osnap.snapkv_scores(_sub(ns, b, ns.q_obs), k, table, P[b:b + 1], w, scale,
                                    pairs=[(0, g)])
        got_c = host(sc[b, g, :n]).astype(np.float64)
        np.testing.assert_allclose(got_c, ref_c[0, g, :n], rtol=1e-4, atol=1e-7)
        # bit-exact selection on the GPU's own scores
        keep = osnap.top_k_positions(osnap.max_pool(got_c, pool), budget - w)
        np.testing.assert_array_equal(g_sel[b, g, : len(keep)], keep)
        # draft over the selected set
        ref, ref_lse = oatt.draft_attention(_sub(ns, b, ns.q_draft), k, v, table, P[b:b + 1] + 1,
                                            g_sel[b:b + 1], g_cnt[b:b + 1], P[b:b + 1] - w, scale,
                                            pairs=[(0, g)])
        hs = slice(g * wl.group, (g + 1) * wl.group)
        assert row_rel_err(host(d_out[b, hs]), ref[0, hs]) <= ATTN_RTOL
        assert lse_err(host(d_lse[b, hs]), ref_lse[0, hs]) <= 1e-4


def test_fullsize_streaming_draft(full):
    ns, wl = full, full.workload
    sink, window = wl.streaming or (16, 496)
    P = ns.prompt_lens_np
    kvd = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_draft, int(P.max()) + 1)
    s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(ns.kv_lens_draft, wl.num_kv_heads, sink, window)
    out, lse = kvss.draft_attn_sparse(kvd, ns.q_draft, s_idx, s_cnt, s_tail, window)
    torch.cuda.synchronize()
    for b, g in _pairs(ns.batch, wl.num_kv_heads):
        k, v, table = subcache(ns, [b])
        ref, _ = oatt.draft_attention(_sub(ns, b, ns.q_draft), k, v, table, P[b:b + 1] + 1,
                                      host(s_idx[b:b + 1]), host(s_cnt[b:b + 1]),
                                      host(s_tail[b:b + 1]), 1 / math.sqrt(wl.head_dim),
                                      pairs=[(0, g)])
        hs = slice(g * wl.group, (g + 1) * wl.group)
        assert row_rel_err(host(out[b, hs]), ref[0, hs]) <= ATTN_RTOL


@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_fullsize_accept(full, temp):
    ns = full
    seed, offset = 4242, 3
    out, n_acc, _ = kvss.spec_accept(ns.target_logits, ns.draft_logits, ns.draft_tokens, temp,
                                     seed, offset)
    torch.cuda.synchronize()
    seqs = sorted({0, ns.batch // 2, ns.batch - 1})
    t = host(ns.target_logits[seqs])
    d = host(ns.draft_logits[seqs])
    x = host(ns.draft_tokens[seqs])
    r_out, r_n = oacc.spec_accept(t, d, x, temp, seed, offset, seq_ids=seqs)
    np.testing.assert_array_equal(host(out[seqs]), r_out)
    np.testing.assert_array_equal(host(n_acc[seqs]), r_n)


def test_fullsize_compact_draft_cache(full):
    """The bench's compact SnapKV draft cache: build, rows bit-exact on sampled pairs, and the
    T = 1 decode over it against the oracle's sparse draft."""
    from oracle.kvcache import compact_rows
    ns, wl = full, full.workload
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    scale = 1 / math.sqrt(wl.head_dim)
    kvp = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, int(P.max()))
    sel, cnt, _ = kvss.snapkv_select(kvp, ns.q_obs, w, pool, budget)
    kvd = kvp.with_lens(ns.kv_lens_draft, int(P.max()) + 1)
    tail = (ns.prompt_lens - w).contiguous()
    B, Hkv, D, bs = ns.batch, wl.num_kv_heads, wl.head_dim, wl.block_size
    cap = budget - w + w + 1
    cb = (cap + bs - 1) // bs
    ck = torch.empty((B * cb, Hkv, bs, D), dtype=ns.k_cache.dtype, device="cuda")
    cv = torch.empty_like(ck)
    ctab = torch.arange(B * cb, dtype=torch.int32, device="cuda").view(B, cb)
    clens = torch.empty(B, dtype=torch.int32, device="cuda")
    kvc = kvss.PagedKV(ck, cv, ctab, clens, cap)
    kvss.kvss_draft_cache_build(kvd, sel, cnt, tail, w + 1, kvc, dst_lens=clens)
    out, lse = kvss.verify_attn_full(kvc, ns.q_draft.unsqueeze(2).contiguous())
    torch.cuda.synchronize()
    g_sel, g_cnt = host(sel), host(cnt)
    np.testing.assert_array_equal(host(clens), g_cnt + w + 1)
    for b, g in _pairs(B, Hkv):
        k, v, table = subcache(ns, [b])
        rk, lens = compact_rows(k, table, P[b:b + 1] + 1, g_sel[b:b + 1], g_cnt[b:b + 1],
                                P[b:b + 1] - w, w + 1)
        n = int(lens[0])
        j = np.arange(n)
        got = host(ck[torch.from_numpy(host(ctab)[b, j // bs]).long().cuda(), g,
                      torch.from_numpy(j % bs).long().cuda()])
        np.testing.assert_array_equal(got, rk[0][g])
        ref, ref_lse = oatt.draft_attention(_sub(ns, b, ns.q_draft), k, v, table, P[b:b + 1] + 1,
                                            g_sel[b:b + 1], g_cnt[b:b + 1], P[b:b + 1] - w, scale,
                                            pairs=[(0, g)])
        hs = slice(g * wl.group, (g + 1) * wl.group)
        assert row_rel_err(host(out[b, hs, 0]), ref[0, hs]) <= ATTN_RTOL
        assert lse_err(host(lse[b, hs, 0]), ref_lse[0, hs]) <= 1e-4


def test_fullsize_topk_draft(full):
    """The bench's dynamic Top-K draft (k = budget - 1) on sampled pairs."""
    ns, wl = full, full.workload
    budget, _, _ = wl.snapkv
    k = budget - 1
    P = ns.prompt_lens_np
    L = P + 1
    scale = 1 / math.sqrt(wl.head_dim)
    kvd = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_draft, int(L.max()))
    sel = torch.empty((ns.batch, wl.num_kv_heads, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(ns.batch, dtype=torch.int32, device="cuda")
    out, lse = kvss.draft_attn_topk(kvd, ns.q_draft, k, sel_idx=sel, sel_count=cnt)
    torch.cuda.synchronize()
    g_sel, g_cnt = host(sel), host(cnt)
    np.testing.assert_array_equal(g_cnt, np.minimum(k, L - 1))
    for b, g in _pairs(ns.batch, wl.num_kv_heads):
        kc, vc, table = subcache(ns, [b])
        q1 = _sub(ns, b, ns.q_draft)
        ref_c = osnap.snapkv_scores(q1[:, :, None, :], kc, table, L[b:b + 1], 1, scale,
                                    pairs=[(0, g)])[0, g, : int(L[b]) - 1]
        r_keep = set(osnap.top_k_positions(ref_c, k).tolist())
        got = set(g_sel[b, g, : g_cnt[b]].tolist())
        diff = got ^ r_keep
        tau = np.sort(ref_c)[::-1][k - 1]
        assert all(abs(ref_c[j] - tau) <= 1e-5 * tau for j in diff), (b, g, sorted(diff)[:5])
        ref, ref_lse = oatt.draft_attention(q1, kc, vc, table, L[b:b + 1], g_sel[b:b + 1],
                                            g_cnt[b:b + 1], L[b:b + 1] - 1, scale, pairs=[(0, g)])
        hs = slice(g * wl.group, (g + 1) * wl.group)
        assert row_rel_err(host(out[b, hs]), ref[0, hs]) <= ATTN_RTOL


@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_fullsize_draft_sample(full, temp):
    ns = full
    logits = ns.draft_logits[:, 0].contiguous()
    tok, _ = kvss.draft_sample(logits, temp, 77, 9, 1)
    torch.cuda.synchronize()
    seqs = sorted({0, ns.batch // 2, ns.batch - 1})
    ref = oacc.draft_sample(host(logits[seqs]).astype(np.float64), temp, 77, 9, 1, seq_ids=seqs)
    np.testing.assert_array_equal(host(tok[seqs]), ref)
