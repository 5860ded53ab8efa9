"""HIP-graph capture of a draft round (sparse draft, decode over a compact cache, draft-token
sampling) replayed several times, with eager work and synchronisations between replays; every
replay must reproduce the eager results bit for bit (the library allocates nothing and issues
no memset, so its calls are capturable)."""

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
