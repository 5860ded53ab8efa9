"""Every call is bitwise repeatable, and the calls that read the paged cache give the same bits
whatever physical blocks hold a sequence's rows.

No call uses float atomics or order-dependent reductions, so a second call on the same inputs
reproduces every output bit. Block placement changes addresses only: the split plan depends
on the lengths and the batch, never on the block table, so a cache whose pages are shuffled
and the same cache copied into an identity layout must agree bit for bit (SnapKV scores and
kept sets, gathered drafts, the dynamic Top-K draft and the compact draft cache built from it).
"""

import ctypes

import numpy as np
import pytest
import torch

from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

CASES = [("qwen32b_ragged", {"batch": 5}), ("llama8b_ctx8k", {"batch": 3}),
         ("tiny_fp32", {})]


def _identity_layout(ns):
    """The same logical cache copied so that sequence b's blocks are consecutive."""
    table = ns.block_table_np
    order = [int(x) for b in range(ns.batch) for x in table[b][table[b] >= 0]]
    idx = torch.tensor(order, dtype=torch.long, device="cuda")
    k2 = ns.k_cache.index_select(0, idx).contiguous()
    v2 = ns.v_cache.index_select(0, idx).contiguous()
    t2 = np.full_like(table, -1)
    nxt = 0
    for b in range(ns.batch):
        nb = int((table[b] >= 0).sum())
        t2[b, :nb] = np.arange(nxt, nxt + nb)
        nxt += nb
    return k2, v2, torch.from_numpy(t2).cuda()


def _run_cache_calls(k, v, table, ns):
    """SnapKV selection, the gathered SnapKV and StreamingLLM drafts, the dynamic Top-K draft
    and the compact draft cache, on one physical layout."""
    wl = ns.workload
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    kv_p = kvss.PagedKV(k, v, table, ns.prompt_lens, int(P.max()))
    kv_d = kvss.PagedKV(k, v, table, ns.kv_lens_draft, int(P.max()) + 1)
    sel, cnt, scores = kvss.snapkv_select(kv_p, ns.q_obs, w, pool, budget, want_scores=True)
    tail = (ns.prompt_lens - w).clamp(min=0).to(torch.int32)
    o_snap, l_snap = kvss.draft_attn_sparse(kv_d, ns.q_draft, sel, cnt, tail, w + 1)
    sink, window = wl.streaming or (16, 496)
    s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(ns.kv_lens_draft, wl.num_kv_heads, sink, window)
    o_str, l_str = kvss.draft_attn_sparse(kv_d, ns.q_draft, s_idx, s_cnt, s_tail, window)
    t_sel = torch.empty((ns.batch, wl.num_kv_heads, budget - 1), dtype=torch.int32, device="cuda")
    t_cnt = torch.empty(ns.batch, dtype=torch.int32, device="cuda")
    o_topk, l_topk = kvss.draft_attn_topk(kv_d, ns.q_draft, budget - 1, sel_idx=t_sel,
                                          sel_count=t_cnt)
    # the compact draft cache (its own identity layout) and a decode over it
    nb = -(-(budget + 1) // wl.block_size)
    shape = (ns.batch * nb,) + tuple(k.shape[1:])
    dk = torch.zeros(shape, dtype=k.dtype, device="cuda")
    dv = torch.zeros(shape, dtype=v.dtype, device="cuda")
    dtab = torch.arange(ns.batch * nb, dtype=torch.int32, device="cuda").view(ns.batch, nb)
    dst = kvss.PagedKV(dk, dv, dtab, torch.zeros(ns.batch, dtype=torch.int32, device="cuda"),
                       nb * wl.block_size)
    d_lens = kvss.kvss_draft_cache_build(kv_d, sel, cnt, tail, w + 1, dst)
    torch.cuda.synchronize()
    return {"sel": sel, "cnt": cnt, "scores": scores, "o_snap": o_snap, "l_snap": l_snap,
            "o_str": o_str, "l_str": l_str, "o_topk": o_topk, "l_topk": l_topk, "t_sel": t_sel,
            "t_cnt": t_cnt, "dk": dk, "dv": dv, "d_lens": d_lens}


def _assert_same(a, b, what):
    for key in a:
        assert torch.equal(a[key], b[key]), f"{what}: {key} differs"


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_cache_calls_repeat_and_ignore_page_order(name, kw):
    torch.manual_seed(0)
    ns = generate(WORKLOADS[name], device="cuda", parts=("attn",), **kw)
    first = _run_cache_calls(ns.k_cache, ns.v_cache, ns.block_table, ns)
    again = _run_cache_calls(ns.k_cache, ns.v_cache, ns.block_table, ns)
    _assert_same(first, again, "repeat")
    k2, v2, t2 = _identity_layout(ns)
    moved = _run_cache_calls(k2, v2, t2, ns)
    _assert_same(first, moved, "identity layout")
    assert int(first["cnt"].min()) >= 0 and int(first["t_cnt"].min()) >= 0


@pytest.mark.parametrize("temp", [0.0, 1.0, 0.3])
def test_samplers_repeat(temp):
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", batch=24, parts=("accept",),
                  vocab=20000)
    runs = []
    for _ in range(2):
        out, n_acc, stats = kvss.spec_accept(ns.target_logits, ns.draft_logits, ns.draft_tokens,
                                             temp, 123, 9, want_stats=True)
        tok, st = kvss.draft_sample(ns.draft_logits[:, 0].contiguous(), temp, 123, 9, 2,
                                    want_stats=True)
        torch.cuda.synchronize()
        runs.append((out, n_acc, stats, tok, st))
    for x, y in zip(*runs):
        assert torch.equal(x, y)


def test_calls_on_a_side_stream_match_the_current_stream():
    """`stream=` runs a call on another stream. The binding allocates the call's outputs and
    workspace (and zero-fills the SnapKV scores) on that stream, so the fills are ordered before
    the kernels, and memory claimed and overwritten on the current stream straight after the
    call cannot be a workspace still in use (the split partials, the SnapKV scores)."""
    torch.manual_seed(0)
    ns = generate(WORKLOADS["llama8b_ctx32k"], device="cuda", parts=("attn",), batch=4,
                  prompt=(20000, 20000))
    wl = ns.workload
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    kv_v = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_verify,
                        int(P.max()) + ns.T)
    kv_p = kv_v.with_lens(ns.prompt_lens, int(P.max()))

    lib = kvss.lib()
    ws_v = lib.kvss_verify_workspace_bytes(ctypes.byref(kv_v.desc()), wl.num_q_heads, ns.T)
    ws_s = lib.kvss_snapkv_workspace_bytes(ctypes.byref(kv_p.desc()), wl.num_q_heads, w, budget)
    assert ws_v > 0 and ws_s > 0

    def churn(nbytes, value):
        # blocks of the size the binding just freed, claimed and overwritten at once
        return [torch.full((nbytes,), value, dtype=torch.uint8, device="cuda") for _ in range(4)]

    def run(stream):
        o, l = kvss.verify_attn_full(kv_v, ns.q_verify, stream=stream)
        held = churn(ws_v, 7)
        sel, cnt, sc = kvss.snapkv_select(kv_p, ns.q_obs, w, pool, budget, want_scores=True,
                                          stream=stream)
        held += churn(ws_s, 3)
        del held
        return o, l, sel, cnt, sc

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    side.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(x, y)
