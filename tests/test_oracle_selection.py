"""Pins of the oracle's draft-set construction: the StreamingLLM sink + window set
(exhaustive set arithmetic) and SnapKV selection (brute-force loops, torch softmax / max_pool1d,
a stable full sort, and the special cases the definition implies)."""

import math

import numpy as np
import pytest
import torch

from oracle.attention import draft_positions
from oracle.snapkv import (max_pool, select_from_scores, snapkv_scores, snapkv_select,
                           top_k_positions)
from oracle.streaming import streaming_positions, streaming_set


@pytest.mark.parametrize("sink,window", [(4, 60), (0, 8), (3, 1), (16, 5)])
def test_streaming_set_exhaustive(sink, window):
    for L in range(0, 81):
        got = streaming_positions(L, sink, window)
        want = [j for j in range(L) if j < sink or j >= L - window]
        assert list(got) == want
        assert len(got) == min(L, sink + window)
        if L > 0:
            assert got[-1] == L - 1                 # the current token is always attended
        sel, cnt, tail = streaming_set([L], 2, sink, window)
        for g in range(2):
            assert list(draft_positions(L, sel[0, g], cnt[0], tail[0])) == want


def test_streaming_budget_at_headline_shape():
    got = streaming_positions(32001, 16, 496)
    assert len(got) == 512 and got[15] == 15 and got[16] == 32001 - 496


def _paged_k(rng, B, Hkv, P, D, bs=16):
    Kl = rng.standard_normal((B, Hkv, P, D))
    nb = (P + bs - 1) // bs
    perm = rng.permutation(B * nb)
    table = perm.reshape(B, nb).astype(np.int32)
    cache = np.zeros((B * nb, Hkv, bs, D))
    for b in range(B):
        for j in range(P):
            cache[table[b, j // bs], :, j % bs] = Kl[b, :, j]
    return Kl, cache, table


def test_scores_brute_force_loops():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, P, D, w = 1, 4, 2, 11, 3, 3
    Kl, kc, table = _paged_k(rng, B, Hkv, P, D, bs=4)
    q_obs = rng.standard_normal((B, Hq, w, D))
    c = snapkv_scores(q_obs, kc, table, [P], w, 0.7)
    G = Hq // Hkv
    for g in range(Hkv):
        for j in range(P - w):
            tot = 0.0
            for h in range(g * G, (g + 1) * G):
                for i in range(w):
                    pos = P - w + i
                    s = [0.7 * sum(q_obs[0, h, i, d] * Kl[0, g, jj, d] for d in range(D))
                         for jj in range(pos + 1)]
                    z = math.fsum(math.exp(x) for x in s)
                    tot += math.exp(s[j]) / z
            assert abs(c[0, g, j] - tot) < 1e-12


def test_scores_match_torch_softmax():
    rng = np.random.default_rng(29)
    B, Hq, Hkv, P, D, w = 2, 8, 2, 70, 16, 16
    Kl, kc, table = _paged_k(rng, B, Hkv, P, D)
    q_obs = rng.standard_normal((B, Hq, w, D))
    c = snapkv_scores(q_obs, kc, table, [P, P], w, 0.25)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            q = torch.from_numpy(q_obs[b, g * G:(g + 1) * G])          # [G, w, D]
            s = 0.25 * q @ torch.from_numpy(Kl[b, g]).T                # [G, w, P]
            pos = torch.arange(P - w, P)[:, None]
            s = s.masked_fill(torch.arange(P)[None, :] > pos, float("-inf"))
            ref = torch.softmax(s, dim=-1).sum(dim=(0, 1))[: P - w]
            np.testing.assert_allclose(c[b, g], ref.numpy(), rtol=1e-12)


def test_pool_matches_torch_max_pool1d():
    rng = np.random.default_rng(31)
    for n in [1, 2, 5, 7, 8, 50]:
        for pool in [1, 3, 7]:
            x = rng.standard_normal(n)
            ref = torch.nn.functional.max_pool1d(torch.from_numpy(x)[None, None], pool, 1,
                                                 padding=pool // 2)[0, 0].numpy()
            np.testing.assert_array_equal(max_pool(x, pool), ref)


def test_topk_matches_stable_sort():
    rng = np.random.default_rng(37)
    for n, k in [(10, 3), (100, 48), (64, 64), (30, 50)]:
        x = rng.integers(0, 6, size=n).astype(np.float64)        # many ties
        order = np.argsort(-x, kind="stable")                    # ties keep index order
        want = np.sort(order[: min(k, n)])
        np.testing.assert_array_equal(top_k_positions(x, k), want)


def test_budget_covering_prompt_selects_everything():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, P, D, w = 2, 4, 2, 40, 8, 8
    _, kc, table = _paged_k(rng, B, Hkv, P, D)
    q_obs = rng.standard_normal((B, Hq, w, D))
    sel, cnt, _ = snapkv_select(q_obs, kc, table, [P, P], w, 7, budget=P, scale=0.3)
    assert list(cnt) == [P - w, P - w]
    np.testing.assert_array_equal(sel[:, :, : P - w], np.tile(np.arange(P - w), (B, Hkv, 1)))
    assert np.all(sel[:, :, P - w:] == -1)


def test_planted_key_and_neighbours_selected():
    rng = np.random.default_rng(43)
    B, Hq, Hkv, P, D, w = 1, 4, 1, 200, 32, 8
    Kl, kc, table = _paged_k(rng, B, Hkv, P, D)
    q_obs = rng.standard_normal((B, Hq, w, D))
    j0 = 77
    direction = q_obs[0].reshape(-1, D).sum(axis=0)               # aligned with every query
    for b in range(B):
        blk, off = table[b, j0 // 16], j0 % 16
        kc[blk, 0, off] = 3.0 * direction / np.linalg.norm(direction) * math.sqrt(D)
    sel, cnt, c = snapkv_select(q_obs, kc, table, [P], w, 7, budget=w + 7, scale=1 / math.sqrt(D))
    assert int(np.argmax(c[0, 0])) == j0
    assert list(sel[0, 0]) == list(range(j0 - 3, j0 + 4))


def test_selection_invariant_to_score_scaling_and_ragged():
    rng = np.random.default_rng(47)
    scores = rng.random((2, 3, 90))
    lens = np.array([90 + 10, 60 + 10])
    a, ca = select_from_scores(scores, lens, 10, 7, 10 + 25)
    b, cb = select_from_scores(scores * 0.125, lens, 10, 7, 10 + 25)    # sum vs mean
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(ca, cb)
    assert list(ca) == [25, 25]
    for bb in range(2):
        for g in range(3):
            row = a[bb, g]
            assert np.all(np.diff(row) > 0) and row.max() < lens[bb] - 10
