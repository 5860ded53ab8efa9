"""GPU parity at the degenerate ends of each call's contract, against the oracle: verify
queries whose causal range is empty or a single key (sequences shorter than T, an empty
cache), drafts over empty, single-key and partly invalid selections (entries past the tail or
the sequence, a negative or over-long tail start), and SnapKV on prompts no longer than the
window, with fewer candidates than the budget, exactly the budget, and one more; and the
acceptance statistics buffer written in full, whatever the temperature."""

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

NAMES = ["llama8b_ctx8k", "tiny_fp32"]


def _inputs(name, batch, prompt):
    torch.manual_seed(0)
    return generate(WORKLOADS[name], device="cuda", parts=("attn",), batch=batch,
                    prompt=(prompt, prompt))


def _check(out, lse, ref, ref_lse, what):
    got, got_lse = host(out), host(lse)
    empty = np.isneginf(ref_lse)
    # an empty attended set gives exactly 0 and -inf
    assert np.all(got[empty] == 0.0), what
    assert np.all(np.isneginf(got_lse[empty])), what
    err = row_rel_err(got, ref)
    print(f"{what}: max row rel err {err:.3e}, empty rows {int(empty.sum())}")
    assert err <= ATTN_RTOL, what
    assert lse_err(got_lse, ref_lse) <= 1e-4, what


@pytest.mark.parametrize("name", NAMES)
def test_verify_short_and_empty_sequences(name):
    ns = _inputs(name, 10, 200)
    wl = ns.workload
    lens = np.array([0, 1, 3, ns.T - 1, ns.T, ns.T + 1, 16, 17, 33, 200 + ns.T], dtype=np.int32)
    t_lens = torch.from_numpy(lens).cuda()
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, t_lens, int(lens.max()))
    out, lse = kvss.verify_attn_full(kv, ns.q_verify)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.verify_attention(host(ns.q_verify), host(ns.k_cache), host(ns.v_cache),
                                         ns.block_table_np, lens, 1 / math.sqrt(wl.head_dim))
    _check(out, lse, ref, ref_lse, f"verify {name}")


@pytest.mark.parametrize("name", NAMES)
def test_draft_degenerate_sets(name):
    ns = _inputs(name, 8, 40)
    wl = ns.workload
    B, Hkv, k_max = 8, wl.num_kv_heads, 8
    L = np.array([40, 40, 40, 0, 1, 40, 40, 40], dtype=np.int32)
    tail_lo = np.array([40, 40, 39, 0, 0, 20, -5, 100], dtype=np.int32)
    count = np.array([0, 1, 8, 0, 0, 8, 3, 8], dtype=np.int32)
    rows = {
        1: [0],
        2: [3, 5, 7, 38, 39, 50, 60, 70],          # 39 (= tail_lo) and beyond are skipped
        5: [1, 2, 4, 8, 9, 15, 18, 19],            # up to tail_lo - 1
        6: [0, 1, 2],                              # tail_lo < 0: every entry skipped
        7: [0, 4, 10, 20, 30, 35, 38, 39],         # tail_lo > L: the list alone
    }
    sel = np.full((B, Hkv, k_max), -1, dtype=np.int32)
    for b, r in rows.items():
        for g in range(Hkv):
            sel[b, g, :len(r)] = r
    t = lambda a: torch.from_numpy(a).cuda()
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, t(L), int(L.max()))
    out, lse = kvss.draft_attn_sparse(kv, ns.q_draft, t(sel), t(count), t(tail_lo), 45)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.draft_attention(host(ns.q_draft), host(ns.k_cache), host(ns.v_cache),
                                        ns.block_table_np, L, sel, count, tail_lo,
                                        1 / math.sqrt(wl.head_dim))
    _check(out, lse, ref, ref_lse, f"draft {name}")
    assert np.isneginf(ref_lse[[0, 3]]).all() and np.isfinite(ref_lse[[1, 2, 4, 5, 6, 7]]).all()


@pytest.mark.parametrize("name", NAMES)
def test_snapkv_short_prompts(name):
    wl = WORKLOADS[name]
    budget, w, pool = wl.snapkv
    k = budget - w
    P = np.array([0, 5, w, w + 1, w + k // 2, w + k, w + k + 1, 3 * budget], dtype=np.int32)
    ns = _inputs(name, len(P), int(P.max()))
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, torch.from_numpy(P).cuda(),
                      int(P.max()))
    sel, cnt, scores = kvss.snapkv_select(kv, ns.q_obs, w, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    g_sel, g_cnt, g_c = host(sel), host(cnt), host(scores)
    n = np.maximum(P - w, 0)
    np.testing.assert_array_equal(g_cnt, np.minimum(n, k))
    for b in range(len(P)):
        if n[b] <= k:                          # every candidate is kept, in order
            for g in range(wl.num_kv_heads):
                np.testing.assert_array_equal(g_sel[b, g, :n[b]], np.arange(n[b]))
                assert np.all(g_sel[b, g, n[b]:] == -1)
    ref_c = osnap.snapkv_scores(host(ns.q_obs), host(ns.k_cache), ns.block_table_np, P, w,
                                1 / math.sqrt(wl.head_dim))
    for b in range(len(P)):
        np.testing.assert_allclose(g_c[b, :, :n[b]], ref_c[b, :, :n[b]], rtol=1e-4, atol=1e-7)
    o_sel, o_cnt = osnap.select_from_scores(g_c.astype(np.float64), P, w, pool, budget)
    np.testing.assert_array_equal(g_sel, o_sel)
    np.testing.assert_array_equal(g_cnt, o_cnt)


@pytest.mark.parametrize("batch", [200, 257])
def test_verify_ragged_batches_longest_first(batch):
    """Ragged batches are taken longest first up to 256 sequences (four 64-sequence chunks of
    the ranking, ties included) and in grid order beyond; every sequence must still land in its
    own output rows."""
    ns = _inputs("llama8b_ctx8k", batch, 300)
    wl = ns.workload
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, 300 + ns.T + 1, size=batch).astype(np.int32)
    lens[::7] = lens[0]                                    # ties
    t_lens = torch.from_numpy(lens).cuda()
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, t_lens, int(lens.max()))
    out, lse = kvss.verify_attn_full(kv, ns.q_verify)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.verify_attention(host(ns.q_verify), host(ns.k_cache), host(ns.v_cache),
                                         ns.block_table_np, lens, 1 / math.sqrt(wl.head_dim))
    _check(out, lse, ref, ref_lse, f"verify ragged B={batch}")


def test_binding_rejects_mismatched_buffers():
    """The binding checks every buffer the kernels index by the call's sizes before launching:
    a wrong shape, dtype or layout raises instead of being read or written out of bounds."""
    ns = _inputs("llama8b_ctx8k", 2, 64)
    wl = ns.workload
    B, Hq, Hkv, T, D = 2, wl.num_q_heads, wl.num_kv_heads, ns.T, wl.head_dim
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_verify, 64 + T)
    f32 = dict(dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    bad = [
        lambda: kvss.verify_attn_full(kv, ns.q_verify, out=torch.empty((B, Hq, T - 1, D), **f32)),
        lambda: kvss.verify_attn_full(kv, ns.q_verify, lse=torch.empty((B, Hq), **f32)),
        lambda: kvss.verify_attn_full(kv, ns.q_verify[:1].contiguous()),
        lambda: kvss.verify_attn_full(kv, ns.q_verify.transpose(1, 2)),
        lambda: kvss.draft_attn_sparse(kv, ns.q_draft, torch.zeros((B, Hkv + 1, 4), **i32),
                                       torch.zeros(B, **i32), torch.zeros(B, **i32), 8),
        lambda: kvss.draft_attn_sparse(kv, ns.q_draft, None, None, torch.zeros(B + 1, **i32), 8),
        lambda: kvss.kvss_streaming_set(ns.kv_lens_draft, Hkv, 4, 60,
                                        sel_idx=torch.zeros((B, Hkv, 3), **i32)),
        lambda: kvss.snapkv_select(kv, torch.zeros((B, Hq, 8, D), dtype=torch.bfloat16, device="cuda"),
                                   8, 3, 16, scores_out=torch.zeros((B, Hkv, 10), **f32)),
        lambda: kvss.spec_accept(torch.zeros((B, 4, 50), **f32), torch.zeros((B, 3, 50), **f32),
                                 torch.zeros((B, 3), **i32), 1.0,
                                 out_tokens=torch.zeros((B, 3), **i32)),
        lambda: kvss.spec_accept(torch.zeros((B, 4, 50), **f32), None, torch.zeros((B, 3), **i32),
                                 1.0),
        lambda: kvss.draft_sample(torch.zeros((B, 50), **f32), 1.0,
                                  tokens=torch.zeros(B, dtype=torch.int64, device="cuda")),
        lambda: kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, torch.zeros(B + 1, **i32), 64),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()


@pytest.mark.parametrize("gamma", [0, 1, 3])
def test_accept_statistics_rows_written_in_full(gamma):
    """Every entry of the caller's statistics buffer is written: at temperature 0 the target
    rows carry only the argmax and the draft rows are zeros; sampling fills every row."""
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", batch=5, parts=("accept",),
                  vocab=3000)
    target = ns.target_logits[:, : gamma + 1].contiguous()
    draft = ns.draft_logits[:, :gamma].contiguous()
    tokens = ns.draft_tokens[:, :gamma].contiguous()
    z = host(target).astype(np.float64)
    for temp in (0.0, 1.0):
        st = torch.full((5, 2 * gamma + 1, 4), float("nan"), dtype=torch.float32, device="cuda")
        kvss.spec_accept(target, draft, tokens, temp, 3, 1, row_stats=st)
        torch.cuda.synchronize()
        s = host(st)
        assert not np.isnan(s).any(), temp
        np.testing.assert_array_equal(s[:, : gamma + 1, 3].astype(np.int64), z.argmax(axis=2))
        if temp == 0:
            assert (s[:, : gamma + 1, :3] == 0).all() and (s[:, gamma + 1:] == 0).all()


def _malformed_rows(B, V, seed):
    """Logit rows [B, V]: all NaN, all -inf, NaN sprinkled over finite values with a tie at the
    maximum, then ordinary rows."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    z = torch.randn((B, V), generator=g) * 2.0
    z[0] = float("nan")
    z[1] = -float("inf")
    z[2, ::7] = float("nan")
    z[2, 11] = z[2, 40] = 50.0
    return z


@pytest.mark.parametrize("V", [1000, 4099])
def test_greedy_argmax_on_malformed_rows(V):
    import oracle.accept as oacc
    B, gamma = 5, 2
    z = _malformed_rows(B, V, 3)
    tok, st = kvss.draft_sample(z.cuda(), 0.0, want_stats=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(tok), oacc.draft_sample(z.numpy(), 0.0))
    assert host(st)[0, 3] == -1.0 and host(tok)[0] == -1
    # greedy acceptance with those rows as target position 0 (draft tokens equal the argmax
    # where one exists, so acceptance reaches position 1)
    t = torch.randn((B, gamma + 1, V)) * 2.0
    t[:, 0] = z
    x = torch.from_numpy(np.stack([[max(oacc.argmax_lowest(z[b].numpy()), 0), 3]
                                   for b in range(B)]).astype(np.int32))
    out, n, rs = kvss.spec_accept(t.cuda(), None, x.cuda(), 0.0, want_stats=True)
    torch.cuda.synchronize()
    r_out, r_n = oacc.greedy_accept(t.numpy(), x.numpy())
    np.testing.assert_array_equal(host(out), r_out)
    np.testing.assert_array_equal(host(n), r_n)
    assert host(rs)[0, 0, 3] == -1.0 and host(out)[0, 0] == -1
