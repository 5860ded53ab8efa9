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
