"""HIP-graph capture of the two sides of a speculative round -- the draft steps (sparse draft,
draft-token sampling) and the verify side (KV append, split verify with its merge, sampling
acceptance) -- replayed several times, with eager work and synchronisations between replays;
every replay must reproduce the eager results bit for bit (the library allocates nothing and
issues no memset, so its calls are capturable)."""

import numpy as np
import pytest
import torch

from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import host

pytestmark = pytest.mark.gpu


def test_draft_round_graph_replays_match_eager():
    torch.manual_seed(0)
    wl = WORKLOADS["llama8b_ctx8k"]
    ns = generate(wl, device="cuda", batch=8, parts=("attn", "accept"), vocab=5000)
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    kvp = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, int(P.max()))
    sel, cnt, _ = kvss.snapkv_select(kvp, ns.q_obs, w, pool, budget)
    kvd = kvp.with_lens(ns.kv_lens_draft, int(P.max()) + 1)
    tail = (ns.prompt_lens - w).contiguous()
    B, Hq, D = ns.batch, wl.num_q_heads, wl.head_dim
    o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(kvss.lib().kvss_draft_workspace_bytes(
        __import__("ctypes").byref(kvd.desc()), Hq, budget - w, w + 1) + 256, dtype=torch.uint8,
        device="cuda")
    logits = ns.draft_logits[:, 0].contiguous()
    toks = torch.empty((4, B), dtype=torch.int32, device="cuda")
    ws_s = torch.empty(kvss.lib().kvss_sample_workspace_bytes(B, logits.shape[1]),
                       dtype=torch.uint8, device="cuda")

    def round_():
        for step in range(4):
            kvss.draft_attn_sparse(kvd, ns.q_draft, sel, cnt, tail, w + 1, out=o, lse=lse, workspace=ws)
            kvss.draft_sample(logits, 1.0, seed=5, offset=11, step=step, tokens=toks[step], workspace=ws_s)

    round_()
    torch.cuda.synchronize()
    ref_o, ref_lse, ref_t = host(o).copy(), host(lse).copy(), host(toks).copy()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        round_()                                   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            round_()
    torch.cuda.synchronize()
    for rep in range(4):
        o.zero_(); lse.zero_(); toks.fill_(-7)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(o), ref_o)
        np.testing.assert_array_equal(host(lse), ref_lse)
        np.testing.assert_array_equal(host(toks), ref_t)
        _ = (ns.q_draft.float() * 2).sum().item()  # unrelated eager kernels and a sync


def test_verify_round_graph_replays_match_eager():
    """The verify side of a round captured as one graph: append the gamma + 1 scored rows,
    verify over the whole cache (split plan with its merge launch), and sampling acceptance
    (statistics, race, finalize). Replays must equal the eager results bit for bit."""
    torch.manual_seed(0)
    wl = WORKLOADS["llama8b_ctx32k"]
    ns = generate(wl, device="cuda", batch=4, parts=("attn", "accept"), vocab=7000,
                  prompt=(20000, 20000))
    P = ns.prompt_lens_np
    B, Hq, Hkv, T, D = ns.batch, wl.num_q_heads, wl.num_kv_heads, ns.T, wl.head_dim
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_verify, int(P.max()) + T)
    gen = torch.Generator(device="cuda").manual_seed(3)
    k_new = torch.randn((B, Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((B, Hkv, T, D), generator=gen, device="cuda").to(torch.bfloat16)
    o = torch.empty((B, Hq, T, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kvss.lib().kvss_verify_workspace_bytes(
        __import__("ctypes").byref(kv.desc()), Hq, T), 256), dtype=torch.uint8, device="cuda")
    V = ns.target_logits.shape[-1]
    ws_a = torch.empty(kvss.lib().kvss_accept_workspace_bytes(B, ns.gamma, V), dtype=torch.uint8,
                       device="cuda")
    out_t = torch.empty((B, T), dtype=torch.int32, device="cuda")
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")

    def round_():
        kvss.kvss_kv_append(kv, k_new, v_new, ns.prompt_lens)
        kvss.verify_attn_full(kv, ns.q_verify, out=o, lse=lse, workspace=ws)
        kvss.spec_accept(ns.target_logits, ns.draft_logits, ns.draft_tokens, 1.0, seed=8, offset=2,
                         out_tokens=out_t, num_accepted=n_acc, workspace=ws_a)

    round_()
    torch.cuda.synchronize()
    ref = [host(x).copy() for x in (o, lse, out_t, n_acc)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        round_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            round_()
    torch.cuda.synchronize()
    for rep in range(4):
        o.zero_(); lse.zero_(); out_t.fill_(-7); n_acc.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, lse, out_t, n_acc), ref):
            np.testing.assert_array_equal(host(got), want)
        _ = (ns.q_verify.float() * 2).sum().item()
