"""GPU parity of every call of the C-ABI library against the fp64 oracle, on seeded inputs.

Reduced-size cases keep each workload's head shape, dtype, gamma, budgets and block layout
(shuffled / ragged where the workload is), with batch cut so the oracle runs in seconds and
contexts long enough to span many tiles, several splits and a ragged final block.
"""

import math

import numpy as np
import pytest
import torch

import oracle.accept as oacc
import oracle.attention as oatt
import oracle.snapkv as osnap
import oracle.streaming as ostream
from oracle.philox import accept_uniform
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import ATTN_RTOL, host, lse_err, row_rel_err

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_fp32", {}),
    ("llama8b_ctx8k", {"batch": 2}),
    ("llama8b_ctx8k", {"batch": 3, "prompt": (37, 37)}),
    ("llama8b_ctx32k", {"batch": 1}),
    ("llama8b_ctx100k", {"batch": 1}),
    ("qwen32b_ragged", {"batch": 3}),
]
IDS = [f"{n}-B{kw.get('batch', 'full')}" + (f"-P{kw['prompt'][0]}" if "prompt" in kw else "")
       for n, kw in CASES]


def _kv(ns, lens, max_len):
    return kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, lens, max_len)


def _inputs(name, kw, parts=("attn",)):
    torch.manual_seed(0)
    return generate(WORKLOADS[name], device="cuda", parts=parts, **kw)


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_verify_matches_oracle(name, kw):
    ns = _inputs(name, kw)
    wl = ns.workload
    P = ns.prompt_lens_np
    kv = _kv(ns, ns.kv_lens_verify, int(P.max()) + ns.T)
    out, lse = kvss.verify_attn_full(kv, ns.q_verify)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.verify_attention(host(ns.q_verify), host(ns.k_cache), host(ns.v_cache),
                                         ns.block_table_np, P + ns.T, 1 / math.sqrt(wl.head_dim))
    err = row_rel_err(host(out), ref)
    print(f"verify {name}: max row rel err {err:.3e}, lse err {lse_err(host(lse), ref_lse):.3e}")
    assert err <= ATTN_RTOL
    assert lse_err(host(lse), ref_lse) <= 1e-4


def _random_selection(ns, k, tail_lo, seed):
    """A seeded ascending selection of k positions from [0, tail_lo[b]) per (b, g)."""
    rng = np.random.default_rng(seed)
    B, Hkv = ns.batch, ns.workload.num_kv_heads
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = min(k, int(tail_lo[b]))
        cnt[b] = n
        for g in range(Hkv):
            sel[b, g, :n] = np.sort(rng.choice(int(tail_lo[b]), size=n, replace=False))
    return sel, cnt


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_draft_matches_oracle(name, kw):
    ns = _inputs(name, kw)
    wl = ns.workload
    P = ns.prompt_lens_np
    L = P + 1
    kv = _kv(ns, ns.kv_lens_draft, int(L.max()))
    scale = 1 / math.sqrt(wl.head_dim)
    qh, kh, vh = host(ns.q_draft), host(ns.k_cache), host(ns.v_cache)
    sets = []
    # StreamingLLM set built by the library's own kernel
    sink, window = wl.streaming or (16, 496)
    s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(ns.kv_lens_draft, wl.num_kv_heads, sink, window)
    sets.append(("streaming", s_idx, s_cnt, s_tail, window))
    # a SnapKV-shaped gathered set: budget - w selected rows + the tail [P - w, L)
    budget, w, _ = wl.snapkv
    tail = np.maximum(P - w, 0).astype(np.int32)
    sel, cnt = _random_selection(ns, budget - w, tail, seed=wl.seed)
    sets.append(("gather", torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(),
                 torch.from_numpy(tail).cuda(), w + 1))
    # a set covering the whole cache: equals plain decode
    sets.append(("full", None, None, torch.zeros(ns.batch, dtype=torch.int32, device="cuda"),
                 int(L.max())))
    for label, si, sc, tl, max_tail in sets:
        out, lse = kvss.draft_attn_sparse(kv, ns.q_draft, si, sc, tl, max_tail)
        torch.cuda.synchronize()
        if si is None:
            ref, ref_lse = oatt.decode_attention(qh, kh, vh, ns.block_table_np, L, scale)
        else:
            ref, ref_lse = oatt.draft_attention(qh, kh, vh, ns.block_table_np, L, host(si), host(sc),
                                                host(tl), scale)
        err = row_rel_err(host(out), ref)
        print(f"draft {name} {label}: max row rel err {err:.3e}")
        assert err <= ATTN_RTOL, label
        assert lse_err(host(lse), ref_lse) <= 1e-4, label


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_streaming_set_bit_exact(name, kw):
    ns = _inputs(name, {**kw}, parts=())
    wl = ns.workload
    sink, window = wl.streaming or (16, 496)
    for lens in (ns.kv_lens_draft, torch.tensor([0, 3, sink, sink + window, sink + window + 1],
                                                dtype=torch.int32, device="cuda")):
        s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(lens, wl.num_kv_heads, sink, window)
        r_idx, r_cnt, r_tail = ostream.streaming_set(host(lens), wl.num_kv_heads, sink, window)
        np.testing.assert_array_equal(host(s_idx), r_idx)
        np.testing.assert_array_equal(host(s_cnt), r_cnt)
        np.testing.assert_array_equal(host(s_tail), r_tail)


@pytest.mark.parametrize("name,kw", CASES, ids=IDS)
def test_snapkv_matches_oracle(name, kw):
    ns = _inputs(name, kw)
    wl = ns.workload
    budget, w, pool = wl.snapkv
    P = ns.prompt_lens_np
    kv = _kv(ns, ns.prompt_lens, int(P.max()))
    sel, cnt, scores = kvss.snapkv_select(kv, ns.q_obs, w, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(wl.head_dim)
    ref_c = osnap.snapkv_scores(host(ns.q_obs), host(ns.k_cache), ns.block_table_np, P, w, scale)
    g_sel, g_cnt, g_c = host(sel), host(cnt), host(scores)
    for b in range(ns.batch):
        n = max(int(P[b]) - w, 0)
        np.testing.assert_allclose(g_c[b, :, :n], ref_c[b, :, :n], rtol=1e-4, atol=1e-7)
    # bit-exact: the oracle's pool + top-k on the GPU's own scores
    o_sel, o_cnt = osnap.select_from_scores(g_c.astype(np.float64), P, w, pool, budget)
    np.testing.assert_array_equal(g_sel, o_sel)
    np.testing.assert_array_equal(g_cnt, o_cnt)
    # against the oracle's own scores: identical except at near-ties of the k-th score
    r_sel, r_cnt = osnap.select_from_scores(ref_c, P, w, pool, budget)
    np.testing.assert_array_equal(g_cnt, r_cnt)
    flips = 0
    for b in range(ns.batch):
        n = max(int(P[b]) - w, 0)
        for g in range(wl.num_kv_heads):
            a = set(g_sel[b, g][g_sel[b, g] >= 0].tolist())
            r = set(r_sel[b, g][r_sel[b, g] >= 0].tolist())
            diff = a ^ r
            if not diff:
                continue
            pooled = osnap.max_pool(ref_c[b, g, :n], pool)
            tau = np.sort(pooled)[::-1][budget - w - 1]
            near = {j for j in diff if abs(pooled[j] - tau) <= 1e-5 * tau}
            assert diff == near, (b, g, sorted(diff - near)[:5])
            flips += len(diff)
    print(f"snapkv {name}: selection flips at near-ties {flips}")


def _stats_decisions(st, tokens, gamma, temp, seed, offset, b):
    """Accept count from the GPU's row statistics, decided in float64 (oracle uniforms)."""
    n = 0
    near = False
    for i in range(gamma):
        t, d = st[i], st[gamma + 1 + i]
        if temp == 0:
            ok = int(t[3]) == int(tokens[i])
        else:
            p = math.exp(float(t[2]) - float(t[0])) / float(t[1])
            q = math.exp(float(d[2]) - float(d[0])) / float(d[1])
            u = accept_uniform(seed, offset, b, i)
            near |= abs(u - p / q) <= 1e-5 * (p / q)
            ok = u < p / q
        if not ok:
            break
        n += 1
    return n, near


@pytest.mark.parametrize("name,batch,vocab", [("tiny_fp32", 2, None), ("llama8b_ctx8k", 6, None),
                                              ("qwen32b_ragged", 4, None),
                                              ("llama8b_ctx32k", 16, 1001)])
@pytest.mark.parametrize("temp", [0.0, 1.0, 0.7, 0.05, 20.0])
def test_accept_matches_oracle(name, batch, vocab, temp):
    ns = generate(WORKLOADS[name], device="cuda", batch=batch, parts=("accept",), vocab=vocab)
    seed, offset = 0x5EED0000 + batch, 17
    out, n_acc, stats = kvss.spec_accept(ns.target_logits, ns.draft_logits, ns.draft_tokens, temp,
                                         seed, offset, want_stats=True)
    torch.cuda.synchronize()
    t, d, x = host(ns.target_logits), host(ns.draft_logits), host(ns.draft_tokens)
    r_out, r_n = oacc.spec_accept(t, d, x, temp, seed, offset)
    g_out, g_n, st = host(out), host(n_acc), host(stats)
    gamma = ns.gamma
    if temp == 0:
        np.testing.assert_array_equal(g_out, r_out)
        np.testing.assert_array_equal(g_n, r_n)
        return
    mism = 0
    for b in range(ns.batch):
        n_st, near = _stats_decisions(st[b], x[b], gamma, temp, seed, offset, b)
        assert n_st == g_n[b] or near, b         # decisions bit-exact given the GPU's statistics
        if (g_out[b] != r_out[b]).any() or g_n[b] != r_n[b]:
            mism += 1
    print(f"accept {name} temp {temp}: sequences differing from the oracle {mism} / {ns.batch}")
    assert mism == 0


def test_verify_is_deterministic_and_layout_free():
    ns = _inputs("qwen32b_ragged", {"batch": 4})
    P = ns.prompt_lens_np
    kv = _kv(ns, ns.kv_lens_verify, int(P.max()) + ns.T)
    o1, l1 = kvss.verify_attn_full(kv, ns.q_verify)
    o2, l2 = kvss.verify_attn_full(kv, ns.q_verify)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the same logical cache laid out with an identity block table gives identical bits
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
    kv2 = kvss.PagedKV(k2, v2, torch.from_numpy(t2).cuda(), ns.kv_lens_verify, int(P.max()) + ns.T)
    o3, l3 = kvss.verify_attn_full(kv2, ns.q_verify)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_verify_independent_of_split_plan():
    """A batch of one and the same sequence inside a larger batch get different split plans:
    at a 20000-key context a single sequence is split 20 ways, a batch of 16 eight ways."""
    ns = _inputs("llama8b_ctx32k", {"batch": 16, "prompt": (20000, 20000)})
    kv = _kv(ns, ns.kv_lens_verify, int(ns.prompt_lens_np.max()) + ns.T)
    full, _ = kvss.verify_attn_full(kv, ns.q_verify)
    one = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table[:1].contiguous(),
                       ns.kv_lens_verify[:1].contiguous(), kv.max_kv_len)
    o1, _ = kvss.verify_attn_full(one, ns.q_verify[:1].contiguous())
    torch.cuda.synchronize()
    assert row_rel_err(host(o1), host(full[:1]).astype(np.float64)) <= 1e-5


@pytest.mark.parametrize("gamma", [0, 1, 2])
@pytest.mark.parametrize("vocab", [64, 9000])
def test_accept_short_speculation_matches_oracle(gamma, vocab):
    """Sampling acceptance at gamma 0-2: gamma = 0 emits only the draw from p_0, which the
    statistics pass races for itself; with planted accepted prefixes and random drafts the
    batch mixes that path with rejections at every position (one or several race slices)."""
    wl = WORKLOADS["llama8b_ctx8k"]
    ns = generate(wl, device="cuda", batch=24, parts=("accept",), vocab=vocab)
    t = ns.target_logits[:, : gamma + 1].contiguous()
    d = ns.draft_logits[:, :gamma].contiguous()
    x = ns.draft_tokens[:, :gamma].contiguous()
    seed, offset = 0xACCE97 + gamma, 5
    for temp in (1.0, 0.6):
        out, n_acc, _ = kvss.spec_accept(t, d, x, temp, seed, offset)
        torch.cuda.synchronize()
        r_out, r_n = oacc.spec_accept(host(t), host(d), host(x), temp, seed, offset)
        np.testing.assert_array_equal(host(n_acc), r_n)
        np.testing.assert_array_equal(host(out), r_out)
        if gamma == 0:
            assert (host(n_acc) == 0).all()
