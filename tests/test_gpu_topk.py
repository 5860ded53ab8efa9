"""GPU parity of the dynamic Top-K draft (draft_attn_topk) against the oracle: the attention
output within the attention bound, the kept positions bit-exact against the same selection run
through snapkv_select, and against the oracle's own set except at near-ties."""

import math

import numpy as np
import pytest
import torch

import oracle.snapkv as osnap
from oracle.attention import decode_attention
from oracle.topk import topk_draft_attention
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import ATTN_RTOL, host, lse_err, row_rel_err

pytestmark = pytest.mark.gpu

CASES = [("tiny_fp32", {}, 48), ("llama8b_ctx8k", {"batch": 2}, 511),
         ("qwen32b_ragged", {"batch": 3}, 1000), ("llama8b_ctx32k", {"batch": 1}, 511)]


@pytest.mark.parametrize("name,kw,k", CASES, ids=[c[0] for c in CASES])
def test_topk_draft_matches_oracle(name, kw, k):
    torch.manual_seed(0)
    ns = generate(WORKLOADS[name], device="cuda", parts=("attn",), **kw)
    wl = ns.workload
    L = ns.prompt_lens_np + 1
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_draft, int(L.max()))
    sel = torch.empty((ns.batch, wl.num_kv_heads, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(ns.batch, dtype=torch.int32, device="cuda")
    out, lse = kvss.draft_attn_topk(kv, ns.q_draft, k, sel_idx=sel, sel_count=cnt)
    # the same selection through the public SnapKV call, with its scores
    q_obs = ns.q_draft.unsqueeze(2).contiguous()
    s_sel, s_cnt, scores = kvss.snapkv_select(kv, q_obs, 1, 1, k + 1, want_scores=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sel), host(s_sel))
    np.testing.assert_array_equal(host(cnt), host(s_cnt))
    # bit-exact: the oracle's top-k on the GPU's own scores
    g_c = host(scores).astype(np.float64)
    o_sel, o_cnt = osnap.select_from_scores(g_c, L, 1, 1, k + 1)
    np.testing.assert_array_equal(host(sel), o_sel)
    np.testing.assert_array_equal(host(cnt), o_cnt)

    scale = 1 / math.sqrt(wl.head_dim)
    ref, ref_lse, r_sel, r_cnt = topk_draft_attention(host(ns.q_draft), host(ns.k_cache),
                                                      host(ns.v_cache), ns.block_table_np, L, k,
                                                      scale)
    np.testing.assert_array_equal(host(cnt), r_cnt)
    flips = 0
    ref_c = osnap.snapkv_scores(host(q_obs), host(ns.k_cache), ns.block_table_np, L, 1, scale)
    for b in range(ns.batch):
        n = int(L[b]) - 1
        for g in range(wl.num_kv_heads):
            a = set(host(sel)[b, g][host(sel)[b, g] >= 0].tolist())
            r = set(r_sel[b, g][r_sel[b, g] >= 0].tolist())
            diff = a ^ r
            if diff:
                tau = np.sort(ref_c[b, g, :n])[::-1][k - 1]
                near = {j for j in diff if abs(ref_c[b, g, j] - tau) <= 1e-5 * tau}
                assert diff == near, (b, g, sorted(diff - near)[:5])
                flips += len(diff)
    print(f"topk {name}: selection flips at near-ties {flips}")
    if flips == 0:
        err = row_rel_err(host(out), ref)
        print(f"topk draft {name}: max row rel err {err:.3e}")
        assert err <= ATTN_RTOL
        assert lse_err(host(lse), ref_lse) <= 1e-4


def test_topk_budget_covering_the_context_is_decode():
    torch.manual_seed(0)
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", parts=("attn",), batch=3,
                  prompt=(200, 900))
    wl = ns.workload
    L = ns.prompt_lens_np + 1
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_draft, int(L.max()))
    out, lse = kvss.draft_attn_topk(kv, ns.q_draft, int(L.max()))
    torch.cuda.synchronize()
    ref, ref_lse = decode_attention(host(ns.q_draft), host(ns.k_cache), host(ns.v_cache),
                                    ns.block_table_np, L, 1 / math.sqrt(wl.head_dim))
    assert row_rel_err(host(out), ref) <= ATTN_RTOL
    assert lse_err(host(lse), ref_lse) <= 1e-4


# Score patterns for both top-k kernels: the one that pools from global memory (more than
# 32 * 1024 candidates, prompts of 40k-45k) and the register-resident one (prompts of 20k-30k).
# Key 0-th coordinates c_j from a few levels and every observation query along the same axis make
# each position's score a function of c_j alone, so equal levels tie exactly.
#   flat        every score equal: the k kept are the lowest positions (the register kernel's
#               prefilter keeps every position, more than fit in LDS: its all-register path)
#   rare_top    a rare top level covering more positions than the budget: ties at the threshold
#   mid_ties    a rarer top level plus a level tied across thousands of positions
#   planted     the generated (peaky) keys with a budget of 1024 (register kernel: groups by
#               position mod 2 within each 32-position run; ties of a pooled maximum split
#               across the budget)
#   planted_2   budget 1500 (register kernel: mod 2, barely enough groups at the shorter prompt)
#   planted_4   budget 2500 (register kernel: groups by position mod 4)
#   big_budget  budget 5000 (register kernel: groups by position mod 8)
#   huge_budget budget 6000 (register kernel: fewer than k groups even mod 8, so no prefilter)
TIE_CASES = [("flat", (1.0,), (0.0,), 512), ("rare_top", (0.004, 0.1, 0.896), (3.0, 1.0, 0.0), 512),
             ("mid_ties", (0.0005, 0.02, 0.9795), (3.0, 1.0, 0.0), 1024),
             ("planted", None, None, 1024), ("planted_2", None, None, 1500),
             ("planted_4", None, None, 2500), ("big_budget", None, None, 5000),
             ("huge_budget", None, None, 6000)]
REGIMES = [("global", (40000, 45000)), ("register", (20000, 30000))]


@pytest.mark.parametrize("regime,prompt", REGIMES, ids=[r[0] for r in REGIMES])
@pytest.mark.parametrize("pattern,probs,levels,budget", TIE_CASES, ids=[c[0] for c in TIE_CASES])
def test_long_context_topk_ties(pattern, probs, levels, budget, regime, prompt):
    torch.manual_seed(0)
    wl = WORKLOADS["llama8b_ctx8k"]
    ns = generate(wl, device="cuda", parts=("attn",), batch=2, prompt=prompt)
    _, w, pool = wl.snapkv
    print(f"\ntopk ties {pattern} ({regime}): prompts {ns.prompt_lens_np.tolist()} budget {budget}",
          flush=True)
    q_obs = ns.q_obs
    if probs is not None:
        rng = np.random.default_rng(7)
        shape = ns.k_cache.shape[:3]
        c = rng.choice(np.asarray(levels, dtype=np.float32), size=shape, p=probs)
        ns.k_cache.zero_()
        ns.k_cache[..., 0] = torch.from_numpy(c).to(ns.k_cache.dtype).cuda()
        q_obs = torch.zeros_like(ns.q_obs)
        q_obs[..., 0] = 8.0
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, ns.max_prompt)
    sel, cnt, scores = kvss.snapkv_select(kv, q_obs, w, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    g_c = host(scores).astype(np.float64)
    o_sel, o_cnt = osnap.select_from_scores(g_c, ns.prompt_lens_np, w, pool, budget)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)
    if pattern == "flat":
        assert (host(sel) == np.arange(budget - w, dtype=np.int32)).all()


# Pool kernels 1 to 9 on both top-k kernels. Over more than 32k candidates (45001-token
# prompts) the global-memory kernel pools through LDS tiles for radii up to 3 and reads its
# neighbours from global memory above; the odd row stride of its pooled workspace leaves most
# (sequence, head) rows not 16-byte aligned (the tile stores then take the range-checked path).
# At 25001 tokens the register kernel takes radii up to 3 and the global-memory kernel radius 4.
@pytest.mark.parametrize("prompt", [45001, 25001])
@pytest.mark.parametrize("pool", [1, 3, 5, 7, 9])
def test_long_context_pool_sizes(pool, prompt):
    torch.manual_seed(0)
    wl = WORKLOADS["llama8b_ctx8k"]
    ns = generate(wl, device="cuda", parts=("attn",), batch=2, prompt=(prompt, prompt))
    _, w, _ = wl.snapkv
    budget = 1024
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, ns.max_prompt)
    sel, cnt, scores = kvss.snapkv_select(kv, ns.q_obs, w, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    assert (ns.max_prompt - w) % 2 == 1
    o_sel, o_cnt = osnap.select_from_scores(host(scores).astype(np.float64), ns.prompt_lens_np, w,
                                            pool, budget)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)
