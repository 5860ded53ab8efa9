"""GPU parity of the cache-maintenance calls (kvss_kv_append, kvss_draft_cache_build) against
the oracle: both are copies, so results must be bit-exact (NaN rows included, compared as
stored bit patterns); the decode over a compact cache must match the sparse draft."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oatt
from oracle.kvcache import append_rows, compact_rows
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate, to_numpy
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import ATTN_RTOL, host, lse_err, row_rel_err

pytestmark = pytest.mark.gpu


def _cache(rng, B, Hkv, D, bs, max_blocks, dtype, spare=5, shuffle=True):
    """Seeded random paged caches (all blocks filled) with a shuffled table and spare blocks."""
    nb = B * max_blocks + spare
    perm = rng.permutation(nb) if shuffle else np.arange(nb)
    table = perm[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    gen = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    k = torch.randn((nb, Hkv, bs, D), generator=gen).to(dtype).cuda()
    v = torch.randn((nb, Hkv, bs, D), generator=gen).to(dtype).cuda()
    return k, v, table


def _bits(t):
    """Stored bits of a device tensor as a host array (bf16 -> uint16, f32 -> uint32)."""
    a = to_numpy(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_append_bit_exact(dtype, D):
    rng = np.random.default_rng(101)
    B, Hkv, bs, mb, T = 6, 8, 16, 6, 5
    k, v, table = _cache(rng, B, Hkv, D, bs, mb, dtype)
    table[2, 5] = k.shape[0] + 3                          # an out-of-range block id
    start = np.array([0, 17, 88, -3, 93, 14], dtype=np.int32)   # 93 + 5 > 96: partly outside
    gen = torch.Generator().manual_seed(7)
    kn = torch.randn((B, Hkv, T, D), generator=gen).to(dtype).cuda()
    vn = torch.randn((B, Hkv, T, D), generator=gen).to(dtype).cuda()
    ref_k, ref_v = append_rows(to_numpy(k), to_numpy(v), table, to_numpy(kn), to_numpy(vn), start)
    kv = kvss.PagedKV(k, v, torch.from_numpy(table).cuda(),
                      torch.zeros(B, dtype=torch.int32, device="cuda"), 0)
    kvss.kvss_kv_append(kv, kn, vn, torch.from_numpy(start).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(k), ref_k.view(_bits(k).dtype))
    np.testing.assert_array_equal(_bits(v), ref_v.view(_bits(v).dtype))


def test_append_verify_tokens_at_batch_64():
    """The gamma + 1 verify rows of a 64-sequence batch appended at ragged lengths."""
    rng = np.random.default_rng(102)
    B, Hkv, D, bs, mb, T = 64, 8, 128, 16, 24, 5
    k, v, table = _cache(rng, B, Hkv, D, bs, mb, torch.bfloat16, spare=0)
    start = rng.integers(0, mb * bs - T + 1, size=B).astype(np.int32)
    gen = torch.Generator().manual_seed(8)
    kn = torch.randn((B, Hkv, T, D), generator=gen).to(torch.bfloat16).cuda()
    vn = torch.randn((B, Hkv, T, D), generator=gen).to(torch.bfloat16).cuda()
    ref_k, ref_v = append_rows(to_numpy(k), to_numpy(v), table, to_numpy(kn), to_numpy(vn), start)
    kv = kvss.PagedKV(k, v, torch.from_numpy(table).cuda(),
                      torch.zeros(B, dtype=torch.int32, device="cuda"), 0)
    kvss.kvss_kv_append(kv, kn, vn, torch.from_numpy(start).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_numpy(k), ref_k)
    np.testing.assert_array_equal(to_numpy(v), ref_v)


def _compact_cache(rng, ns, cap, dtype):
    """An empty compact cache for `cap` slots per sequence with a shuffled block table."""
    bs = 16
    cb = (cap + bs - 1) // bs
    B, Hkv, D = ns.batch, ns.workload.num_kv_heads, ns.workload.head_dim
    perm = rng.permutation(B * cb).astype(np.int32)
    table = perm.reshape(B, cb)
    k = torch.zeros((B * cb, Hkv, bs, D), dtype=dtype, device="cuda")
    v = torch.zeros_like(k)
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    return kvss.PagedKV(k, v, torch.from_numpy(table).cuda(), lens, cap), table


def _compare_compact(dst, dst_table, dst_lens, ns, L, sel, cnt, tail, max_tail):
    kh, vh = host(ns.k_cache), host(ns.v_cache)
    rk, lens = compact_rows(kh, ns.block_table_np, L, sel, cnt, tail, max_tail)
    rv, _ = compact_rows(vh, ns.block_table_np, L, sel, cnt, tail, max_tail)
    np.testing.assert_array_equal(host(dst_lens), lens)
    gk, gv = host(dst.k), host(dst.v)
    bs = gk.shape[2]
    for b in range(ns.batch):
        j = np.arange(int(lens[b]))
        blk = dst_table[b, j // bs]
        np.testing.assert_array_equal(gk[blk, :, j % bs].transpose(1, 0, 2), rk[b])
        np.testing.assert_array_equal(gv[blk, :, j % bs].transpose(1, 0, 2), rv[b])


def _selection(rng, B, Hkv, k, tail_lo):
    sel = np.full((B, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = min(k, int(tail_lo[b]))
        cnt[b] = n
        for g in range(Hkv):
            sel[b, g, :n] = np.sort(rng.choice(int(tail_lo[b]), size=n, replace=False))
    return sel, cnt


@pytest.mark.parametrize("name,kw", [("llama8b_ctx8k", {"batch": 3}),
                                     ("qwen32b_ragged", {"batch": 3}),
                                     ("tiny_fp32", {})])
def test_compact_build_and_decode(name, kw):
    """Compact SnapKV-shaped draft cache: bit-exact rows; a T = 1 verify over it equals the
    sparse draft over the original cache."""
    torch.manual_seed(0)
    ns = generate(WORKLOADS[name], device="cuda", parts=("attn",), **kw)
    wl = ns.workload
    rng = np.random.default_rng(wl.seed + 7)
    P = ns.prompt_lens_np
    L = P + 1
    budget, w, _ = wl.snapkv
    k = budget - w
    tail = np.maximum(P - w, 0).astype(np.int32)
    sel, cnt = _selection(rng, ns.batch, wl.num_kv_heads, k, tail)
    src = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_draft, int(L.max()))
    dst, dst_table = _compact_cache(rng, ns, k + w + 1, ns.k_cache.dtype)
    t_sel, t_cnt, t_tail = (torch.from_numpy(x).cuda() for x in (sel, cnt, tail))
    dst_lens = kvss.kvss_draft_cache_build(src, t_sel, t_cnt, t_tail, w + 1, dst)
    torch.cuda.synchronize()
    _compare_compact(dst, dst_table, dst_lens, ns, L, sel, cnt, tail, w + 1)

    scale = 1 / math.sqrt(wl.head_dim)
    kvc = dst.with_lens(dst_lens, k + w + 1)
    out, lse = kvss.verify_attn_full(kvc, ns.q_draft.unsqueeze(2).contiguous())
    g_out, g_lse = kvss.draft_attn_sparse(src, ns.q_draft, t_sel, t_cnt, t_tail, w + 1)
    torch.cuda.synchronize()
    ref, ref_lse = oatt.draft_attention(host(ns.q_draft), host(ns.k_cache), host(ns.v_cache),
                                        ns.block_table_np, L, sel, cnt, tail, scale)
    err = row_rel_err(host(out)[:, :, 0], ref)
    print(f"compact decode {name}: max row rel err {err:.3e}")
    assert err <= ATTN_RTOL
    assert lse_err(host(lse)[:, :, 0], ref_lse) <= 1e-4
    # the two GPU paths read the same rows; only the summation order differs
    assert row_rel_err(host(out)[:, :, 0], host(g_out)) <= 1e-5


def test_compact_build_streaming_and_edge_cases():
    """StreamingLLM sink list, no list at all (k_max = 0), listed positions the compact cache
    cannot hold, an over-long tail, and a destination block id out of range."""
    torch.manual_seed(0)
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", parts=("attn",), batch=4,
                  prompt=(300, 700))
    wl = ns.workload
    rng = np.random.default_rng(55)
    P = ns.prompt_lens_np
    L = P + 1
    src = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_draft, int(L.max()))
    # StreamingLLM: sink 16 + window 128
    s_idx, s_cnt, s_tail = kvss.kvss_streaming_set(ns.kv_lens_draft, wl.num_kv_heads, 16, 128)
    dst, dst_table = _compact_cache(rng, ns, 16 + 128, ns.k_cache.dtype)
    lens = kvss.kvss_draft_cache_build(src, s_idx, s_cnt, s_tail, 128, dst)
    torch.cuda.synchronize()
    _compare_compact(dst, dst_table, lens, ns, L, host(s_idx), host(s_cnt), host(s_tail), 128)
    # no list: the compact cache is the tail alone
    tail = (L - 40).astype(np.int32)
    dst, dst_table = _compact_cache(rng, ns, 40, ns.k_cache.dtype)
    lens = kvss.kvss_draft_cache_build(src, None, None, torch.from_numpy(tail).cuda(), 40, dst)
    torch.cuda.synchronize()
    empty = np.zeros((ns.batch, wl.num_kv_heads, 0), dtype=np.int32)
    _compare_compact(dst, dst_table, lens, ns, L, empty, np.zeros(ns.batch, np.int32), tail, 40)
    # invalid listed entries (>= tail_lo, negative) and a tail longer than max_tail (seq 3)
    tail = np.array([200, 250, 280, 100], dtype=np.int32)
    sel, cnt = _selection(rng, ns.batch, wl.num_kv_heads, 20, tail)
    sel[0, 1, 3] = tail[0] + 5
    sel[1, 0, 0] = -4
    max_tail = int((L[:3] - tail[:3]).max())
    assert L[3] - tail[3] > max_tail
    dst, dst_table = _compact_cache(rng, ns, 20 + max_tail, ns.k_cache.dtype)
    lens = kvss.kvss_draft_cache_build(src, torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(),
                                       torch.from_numpy(tail).cuda(), max_tail, dst)
    torch.cuda.synchronize()
    _compare_compact(dst, dst_table, lens, ns, L, sel, cnt, tail, max_tail)
    assert np.isnan(host(dst.k.float())[dst_table[3, 0], 0, 0]).all()
    # a destination block id out of range: those slots are skipped, the rest is written
    bad_table = dst_table.copy()
    bad_table[2, 0] = dst.num_blocks + 9
    dst2 = kvss.PagedKV(torch.zeros_like(dst.k), torch.zeros_like(dst.v),
                        torch.from_numpy(bad_table).cuda(), dst.kv_lens, dst.max_kv_len)
    kvss.kvss_draft_cache_build(src, torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(),
                                torch.from_numpy(tail).cuda(), max_tail, dst2)
    torch.cuda.synchronize()
    g2, g1 = host(dst2.k), host(dst.k)
    for b in range(ns.batch):
        for blk_i in range(bad_table.shape[1]):
            if b == 2 and blk_i == 0:
                continue
            np.testing.assert_array_equal(g2[bad_table[b, blk_i]], g1[dst_table[b, blk_i]])
