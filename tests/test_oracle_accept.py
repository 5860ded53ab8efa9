"""Pins of the oracle's acceptance step and its Philox generator.

* Philox4x32-10 against the published known-answer vectors (tests/golden).
* The acceptance rule against the exact Leviathan identity, enumerated analytically on tiny
  vocabularies, and the oracle's Philox-driven sampler against it statistically (chi-square on
  emitted tokens; the mean emitted count against MagicDec Eq. (1)).
* Greedy acceptance against a direct enumeration of matching prefixes.
"""

import itertools
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle.accept import (argmax_lowest, draft_sample, exponential_race, greedy_accept, rejection_accept,
                           rejection_accept_one, softmax)
from oracle.philox import accept_uniform, draft_uniforms, philox4x32_10, race_uniforms, to_uniform

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        vals = [int(x, 16) for x in r]
        got = philox4x32_10(vals[0:4], vals[4:6])
        assert [int(x) for x in got] == vals[6:10]


def test_uniform_mapping_exact_in_float32():
    x = np.array([0, 1, 511, 512, 2**31, 2**32 - 1], dtype=np.uint64)
    u = to_uniform(x)
    assert np.all((u > 0) & (u < 1))
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
    assert u[0] == 2.0 ** -24 and u[-1] == 1 - 2.0 ** -24
    # the race uniforms of token x are word x % 4 of block x // 4
    r = race_uniforms(5, 9, 2, 3, 10)
    w = philox4x32_10((2, (1 << 16) | 3, 2, 9), (5, 0))
    assert r[9] == to_uniform(w[1]) and r.shape == (10,)
    w0 = philox4x32_10((0, 1, 2, 9), (5, 0))
    assert accept_uniform(5, 9, 2, 1) == to_uniform(w0[0])


def _leviathan_first_token(p, q):
    """Exact law of the token emitted at a position: accept x ~ q w.p. min(1, p/q), else draw
    from norm(max(0, p - q))."""
    res = np.maximum(p - q, 0)
    res = res / res.sum() if res.sum() > 0 else p
    law = np.zeros_like(p)
    for x in range(p.shape[0]):
        a = min(1.0, p[x] / q[x])
        law[x] += q[x] * a
        law += q[x] * (1 - a) * res
    return law


def test_leviathan_identity_exhaustive():
    """Enumerating every draft sequence on tiny vocabularies: each emitted position has law p_i
    and the emitted count follows the product of per-position acceptance masses."""
    rng = np.random.default_rng(53)
    for V in (2, 3, 5, 8):
        for gamma in (1, 2, 3):
            p = np.stack([softmax(rng.standard_normal(V) * 1.4, 1.0) for _ in range(gamma + 1)])
            q = np.stack([softmax(rng.standard_normal(V) * 1.4, 1.0) for _ in range(gamma)])
            for i in range(gamma):
                np.testing.assert_allclose(_leviathan_first_token(p[i], q[i]), p[i], atol=1e-12)
            # probability of reaching each position, by enumerating draft sequences
            reach = np.zeros(gamma + 1)
            for xs in itertools.product(range(V), repeat=gamma):
                w = 1.0
                reach[0] += np.prod([q[i, xs[i]] for i in range(gamma)])
                for k in range(gamma):
                    w *= min(1.0, p[k, xs[k]] / q[k, xs[k]])
                    reach[k + 1] += np.prod([q[i, xs[i]] for i in range(gamma)]) * w
            alpha = np.minimum(p[:gamma], q).sum(axis=1)
            np.testing.assert_allclose(reach, np.concatenate([[1.0], np.cumprod(alpha)]),
                                       atol=1e-12)


def test_accept_threshold_direction():
    """The decision is u < p(x) / q(x): a grid of uniforms accepts a fraction min(1, p/q)."""
    p = np.array([[0.1, 0.6, 0.3], [0.2, 0.2, 0.6]])
    q = np.array([[0.4, 0.3, 0.3]])
    grid = (np.arange(4096) + 0.5) / 4096
    for x, want in [(0, 0.25), (1, 1.0), (2, 1.0)]:
        acc = [rejection_accept_one(p, q, [x], lambda i, u=u: u,
                                    lambda i: np.full(3, 0.5))[1] for u in grid]
        assert abs(np.mean(acc) - want) < 1.0 / 4096


def test_exponential_race_law():
    rng = np.random.default_rng(59)
    w = np.array([0.0, 1.0, 3.0, 0.5, 0.0, 2.5])
    draws = np.array([exponential_race(w, rng.random(6)) for _ in range(40000)])
    assert not np.isin(draws, [0, 4]).any()
    counts = np.bincount(draws, minlength=6)[[1, 2, 3, 5]]
    exp = 40000 * w[[1, 2, 3, 5]] / w.sum()
    assert stats.chisquare(counts, exp).pvalue > 1e-4


def test_rejection_sampler_statistics_and_eq1():
    """The oracle's full Philox-driven path: emitted tokens follow the target law at every
    position, and with equal per-position acceptance mass alpha the mean emitted count is
    Omega(gamma, alpha) = (1 - alpha^(gamma+1)) / (1 - alpha) (MagicDec Eq. (1))."""
    rng = np.random.default_rng(61)
    V, gamma, N = 6, 3, 30000
    zt = rng.standard_normal(V) * 1.4
    zd = rng.standard_normal(V) * 1.4
    p, q = softmax(zt, 1.0), softmax(zd, 1.0)
    target = np.tile(zt, (N, gamma + 1, 1))
    draft = np.tile(zd, (N, gamma, 1))
    tokens = rng.choice(V, size=(N, gamma), p=q)            # drafts sampled from q
    out, n_acc = rejection_accept(target, draft, tokens, 1.0, seed=0x1234ABCD5678, offset=7)
    alpha = np.minimum(p, q).sum()
    omega = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    emitted = (out >= 0).sum(axis=1)
    assert np.all(emitted == n_acc + 1)
    se = emitted.std() / math.sqrt(N)
    assert abs(emitted.mean() - omega) < 4.5 * se
    for k in range(gamma + 1):
        col = out[:, k][out[:, k] >= 0]
        counts = np.bincount(col, minlength=V)
        assert stats.chisquare(counts, col.size * p).pvalue > 1e-4
    # accepted drafts are emitted verbatim
    for b in range(200):
        assert list(out[b, : n_acc[b]]) == list(tokens[b, : n_acc[b]])


def test_rejection_temperature_scales_logits():
    rng = np.random.default_rng(67)
    t = rng.standard_normal((3, 4, 9))
    d = rng.standard_normal((3, 3, 9))
    x = rng.integers(0, 9, (3, 3))
    a = rejection_accept(t, d, x, 0.5, seed=3, offset=1)
    b = rejection_accept(t * 2.0, d * 2.0, x, 1.0, seed=3, offset=1)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_greedy_enumeration():
    rng = np.random.default_rng(71)
    V, gamma = 3, 2
    target = rng.standard_normal((1, gamma + 1, V))
    target[0, 1, :] = [0.5, 0.5, -1.0]                      # a tie: lowest id wins
    best = [argmax_lowest(target[0, i]) for i in range(gamma + 1)]
    assert best[1] == 0
    for xs in itertools.product(range(V), repeat=gamma):
        out, n = greedy_accept(target, np.array([xs]))
        k = 0
        while k < gamma and xs[k] == best[k]:
            k += 1
        assert n[0] == k
        assert list(out[0, :k + 1]) == list(xs[:k]) + [best[k]]
        assert np.all(out[0, k + 1:] == -1)


def test_draft_sample_greedy_is_argmax():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((6, 40))
    logits[2, [5, 17]] = 10.0                     # a tie: the lower id wins
    np.testing.assert_array_equal(draft_sample(logits, 0.0),
                                  [int(np.flatnonzero(r == r.max())[0]) for r in logits])


def test_draft_sample_law():
    """Across offsets the sampled tokens follow softmax(logits / t) (chi-square)."""
    z = np.array([[1.0, 0.2, -0.5, 2.0, 0.0, -1.5]])
    t = 0.8
    p = np.exp(z[0] / t - (z[0] / t).max())
    p /= p.sum()
    n = 20000
    draws = np.array([draft_sample(z, t, seed=77, offset=o, step=2)[0] for o in range(n)])
    counts = np.bincount(draws, minlength=z.shape[1])
    assert stats.chisquare(counts, p * n).pvalue > 1e-3


def test_draft_stream_is_independent_of_the_acceptance_race():
    """Same (seed, offset, sequence, position): the draft and race streams draw different words."""
    u_race = race_uniforms(5, 3, 1, 2, 64)
    u_draft = draft_uniforms(5, 3, 1, 2, 64)
    assert not np.any(u_race == u_draft)
    assert abs(np.corrcoef(u_race, u_draft)[0, 1]) < 0.4


def test_argmax_over_non_nan_entries():
    """Reading of argmax on malformed rows: NaN entries are skipped (lowest index of the maximum
    of the rest); a row of -inf has its maximum at every entry, so index 0; a row of NaN has no
    argmax (-1). Brute force over small rows with NaN / -inf / ties placed at every position."""
    inf = np.inf
    assert argmax_lowest([-inf] * 5) == 0
    assert argmax_lowest([np.nan, np.nan]) == -1
    assert argmax_lowest([1.0, np.nan, 3.0, 3.0]) == 2
    assert argmax_lowest([np.nan, -inf, -2.0]) == 2
    rng = np.random.default_rng(7)
    for _ in range(500):
        n = int(rng.integers(1, 9))
        z = rng.choice([-inf, -1.0, 0.0, 2.0, np.nan], size=n)
        ok = [i for i in range(n) if not math.isnan(z[i])]
        want = -1 if not ok else min(i for i in ok if z[i] == max(z[j] for j in ok))
        assert argmax_lowest(z) == want


def test_greedy_accept_on_a_row_without_argmax():
    """A target row of NaN has argmax -1: the draft token there is rejected and -1 emitted."""
    t = np.zeros((1, 3, 4))
    t[0, 0, 2] = 5.0
    t[0, 1, :] = np.nan
    out, n = greedy_accept(t, np.array([[2, 1]], dtype=np.int32))
    assert n.tolist() == [1] and out.tolist() == [[2, -1, -1]]
    assert draft_sample(np.array([[np.nan, np.nan], [-np.inf, -np.inf]]), 0.0).tolist() == [-1, 0]


def test_rejection_accept_without_drafts_is_one_draw_from_p0():
    """gamma = 0 (Section 3.1 with no speculation): nothing to accept, one token emitted by the
    exponential race over p_0 with the race uniforms of position 0."""
    rng = np.random.default_rng(11)
    B, V = 3, 50
    target = rng.normal(size=(B, 1, V)) * 2.0
    draft = np.zeros((B, 0, V))
    tokens = np.zeros((B, 0), dtype=np.int32)
    out, n = rejection_accept(target, draft, tokens, 0.8, seed=9, offset=2)
    assert (n == 0).all() and out.shape == (B, 1)
    for b in range(B):
        p = softmax(target[b, 0], 0.8)
        assert out[b, 0] == exponential_race(p, race_uniforms(9, 2, b, 0, V))
