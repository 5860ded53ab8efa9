"""GPU parity of the attention and SnapKV calls at softmax scales other than 1/sqrt(D): a large
scale (peaky softmax: the running maximum moves by many units, exercising the rescale of the
lazy reference) and a negative scale (SnapKV folds the sign into its staged queries)."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oatt
import oracle.snapkv as osnap
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import ATTN_RTOL, host, lse_err, row_rel_err

pytestmark = pytest.mark.gpu

SCALES = [0.5, -0.04]


def _setup(batch=2, prompt=(900, 1500)):
    torch.manual_seed(0)
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", parts=("attn",), batch=batch,
                  prompt=prompt)
    P = ns.prompt_lens_np
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.prompt_lens, int(P.max()))
    return ns, P, kv


@pytest.mark.parametrize("scale", SCALES)
def test_verify_and_decode_at_scale(scale):
    ns, P, kv = _setup()
    kv_v = kv.with_lens(ns.kv_lens_verify, int(P.max()) + ns.T)
    out, lse = kvss.verify_attn_full(kv_v, ns.q_verify, scale=scale)
    d_out, d_lse = kvss.verify_attn_full(kv_v, ns.q_verify[:, :, -1:].contiguous(), scale=scale)
    torch.cuda.synchronize()
    k, v = host(ns.k_cache), host(ns.v_cache)
    ref, ref_lse = oatt.verify_attention(host(ns.q_verify), k, v, ns.block_table_np, P + ns.T, scale)
    assert row_rel_err(host(out), ref) <= ATTN_RTOL
    assert lse_err(host(lse), ref_lse) <= 1e-4
    ref_d, ref_dl = oatt.decode_attention(host(ns.q_verify)[:, :, -1], k, v, ns.block_table_np,
                                          P + ns.T, scale)
    assert row_rel_err(host(d_out)[:, :, 0], ref_d) <= ATTN_RTOL
    assert lse_err(host(d_lse)[:, :, 0], ref_dl) <= 1e-4


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("w", [2, 32], ids=["stored", "mfma"])
def test_snapkv_at_scale(scale, w):
    ns, P, kv = _setup()
    q_obs = ns.q_obs[:, :, -w:].contiguous()
    budget, pool = 64 + w, 7
    sel, cnt, scores = kvss.snapkv_select(kv, q_obs, w, pool, budget, scale=scale, want_scores=True)
    torch.cuda.synchronize()
    ref_c = osnap.snapkv_scores(host(q_obs), host(ns.k_cache), ns.block_table_np, P, w, scale)
    g_c = host(scores)
    for b in range(ns.batch):
        n = int(P[b]) - w
        np.testing.assert_allclose(g_c[b, :, :n], ref_c[b, :, :n], rtol=1e-4, atol=1e-7)
    o_sel, o_cnt = osnap.select_from_scores(g_c.astype(np.float64), P, w, pool, budget)
    np.testing.assert_array_equal(host(sel), o_sel)
    np.testing.assert_array_equal(host(cnt), o_cnt)
