"""Pins of the oracle's dynamic Top-K draft against brute force: for one query head per KV
head the kept set is the top-k raw scores; for a group it is the top-k of the summed per-head
softmax probabilities (torch softmax); k >= L - 1 keeps everything (= plain decode)."""

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention
from oracle.topk import topk_draft_attention, topk_positions

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _cache(rng, B, Hkv, L_max, bs, D):
    nb = (L_max + bs - 1) // bs
    perm = rng.permutation(B * nb)
    table = perm.reshape(B, nb).astype(np.int32)
    k = rng.standard_normal((B * nb, Hkv, bs, D))
    v = rng.standard_normal((B * nb, Hkv, bs, D))
    return k, v, table


def _logical(cache, table, b, g, n):
    bs = cache.shape[2]
    return np.stack([cache[table[b, j // bs], g, j % bs] for j in range(n)])


def _top(scores, k):
    """Indices of the k largest scores, ties to the lower index, ascending (stable sort)."""
    order = np.argsort(-scores, kind="stable")
    return np.sort(order[:k])


def test_single_head_keeps_the_top_raw_scores():
    rng = np.random.default_rng(3)
    B, Hkv, D, bs, k = 3, 2, 8, 4, 5
    L = np.array([23, 9, 17])
    kc, vc, table = _cache(rng, B, Hkv, 24, bs, D)
    q = rng.standard_normal((B, Hkv, D))                     # G = 1
    # force an exact tie between two candidate keys of (0, 0)
    kc[table[0, 1], 0, 2] = kc[table[0, 0], 0, 3]
    sel, cnt, _ = topk_positions(q, kc, table, L, k, 0.3)
    for b in range(B):
        assert cnt[b] == min(k, L[b] - 1)
        for g in range(Hkv):
            K = _logical(kc, table, b, g, L[b] - 1)
            expect = _top(K @ q[b, g], k)
            np.testing.assert_array_equal(sel[b, g, :cnt[b]], expect)


def test_group_keeps_the_top_summed_probabilities():
    rng = np.random.default_rng(4)
    B, Hkv, G, D, bs, k = 2, 2, 3, 16, 4, 6
    L = np.array([31, 20])
    kc, vc, table = _cache(rng, B, Hkv, 32, bs, D)
    q = rng.standard_normal((B, Hkv * G, D))
    scale = 0.25
    sel, cnt, _ = topk_positions(q, kc, table, L, k, scale)
    for b in range(B):
        for g in range(Hkv):
            K = torch.from_numpy(_logical(kc, table, b, g, L[b]))      # includes the current key
            s = scale * (torch.from_numpy(q[b, g * G:(g + 1) * G]) @ K.T)
            p = torch.softmax(s, dim=-1).sum(0).numpy()[: L[b] - 1]
            np.testing.assert_array_equal(sel[b, g, :cnt[b]], _top(p, k))


def test_budget_covering_the_context_is_plain_decode():
    rng = np.random.default_rng(5)
    B, Hkv, G, D, bs = 2, 2, 2, 8, 4
    L = np.array([12, 7])
    kc, vc, table = _cache(rng, B, Hkv, 12, bs, D)
    q = rng.standard_normal((B, Hkv * G, D))
    out, lse, sel, cnt = topk_draft_attention(q, kc, vc, table, L, 20, 0.4)
    ref, ref_lse = decode_attention(q, kc, vc, table, L, 0.4)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(cnt, L - 1)
