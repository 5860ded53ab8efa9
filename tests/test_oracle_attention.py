"""Pins of the oracle's attention (verify / decode / sparse draft) against things other than
itself: torch's scaled_dot_product_attention in float64, brute-force loops, closed forms and
the invariants the paper's setting implies (verify = sequential decodes; a full draft set =
decode; split-softmax merging)."""

import math

import numpy as np
import pytest
import torch

from oracle.attention import (attend, decode_attention, draft_attention, draft_positions,
                              merge_partials, softmax_partial, verify_attention)
from oracle.kvcache import as_f64

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _paged(logical, block_size, rng, shuffle=True):
    """Scatter logical per-sequence rows [B, Hkv, L, D] into a paged cache (test side)."""
    B, Hkv, L, D = logical.shape
    nb = (L + block_size - 1) // block_size
    total = B * nb
    perm = rng.permutation(total) if shuffle else np.arange(total)
    table = perm.reshape(B, nb).astype(np.int32)
    cache = np.zeros((total, Hkv, block_size, D), dtype=logical.dtype)
    for b in range(B):
        for j in range(L):
            cache[table[b, j // block_size], :, j % block_size, :] = logical[b, :, j, :]
    return cache, table


def _sdpa(q, K, V, mask, scale):
    """torch SDPA in float64 on CPU; q [R, D], K/V [n, D], mask bool [R, n]."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    mt = torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt,
                                                            scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("B,Hq,Hkv,T,D,L,bs", [(2, 8, 2, 4, 64, 77, 16), (3, 10, 2, 5, 32, 40, 8),
                                               (1, 4, 4, 1, 16, 19, 16)])
def test_verify_matches_torch_sdpa(B, Hq, Hkv, T, D, L, bs):
    rng = np.random.default_rng(7)
    G = Hq // Hkv
    Kl = rng.standard_normal((B, Hkv, L, D))
    Vl = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hq, T, D))
    kc, table = _paged(Kl, bs, rng)
    vc = np.zeros_like(kc)
    for b in range(B):                                 # V shares K's block table
        for j in range(L):
            vc[table[b, j // bs], :, j % bs, :] = Vl[b, :, j, :]
    lens = np.full(B, L)
    scale = 1.0 / math.sqrt(D)
    out, lse = verify_attention(q, kc, vc, table, lens, scale)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            mask = np.arange(L)[None, :] <= (L - T + np.arange(T))[:, None]
            ref = _sdpa(q[b, h], Kl[b, g], Vl[b, g], mask, scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)
            s = scale * q[b, h] @ Kl[b, g].T
            s = np.where(mask, s, -np.inf)
            ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
            np.testing.assert_allclose(lse[b, h], ref_lse, rtol=1e-12)


def test_attend_brute_force_loops():
    rng = np.random.default_rng(3)
    R, n, D = 3, 9, 5
    q = rng.standard_normal((R, D))
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    limits = np.array([0, 4, 8])
    out, lse = attend(q, K, V, 0.37, limits)
    for r in range(R):
        s = [0.37 * math.fsum(q[r, d] * K[j, d] for d in range(D)) for j in range(limits[r] + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        for d in range(D):
            assert abs(out[r, d] - math.fsum(w[j] * V[j, d] for j in range(len(s))) / z) < 1e-13
        assert abs(lse[r] - (m + math.log(z))) < 1e-13


def test_closed_forms():
    rng = np.random.default_rng(5)
    D, n = 8, 13
    q = rng.standard_normal((1, D))
    k = rng.standard_normal(D)
    V = rng.standard_normal((n, D))
    # all keys equal: uniform weights, output = mean of attended rows, lse = s + log n
    out, lse = attend(q, np.tile(k, (n, 1)), V, 0.5)
    np.testing.assert_allclose(out[0], V.mean(axis=0), rtol=1e-13, atol=1e-14)
    assert abs(lse[0] - (0.5 * q[0] @ k + math.log(n))) < 1e-12
    # a single attended key: output = that value row
    K = rng.standard_normal((n, D))
    out, _ = attend(q, K, V, 0.5, limits=[0])
    np.testing.assert_allclose(out[0], V[0], rtol=0, atol=0)
    # constant value rows: output = that constant
    c = rng.standard_normal(D)
    out, _ = attend(q, K, np.tile(c, (n, 1)), 0.5)
    np.testing.assert_allclose(out[0], c, rtol=1e-13)


def _cache(rng, B, Hkv, L, D, bs=16):
    Kl = rng.standard_normal((B, Hkv, L, D))
    Vl = rng.standard_normal((B, Hkv, L, D))
    kc, table = _paged(Kl, bs, rng)
    vc = np.zeros_like(kc)
    for b in range(B):
        for j in range(L):
            vc[table[b, j // bs], :, j % bs, :] = Vl[b, :, j, :]
    return kc, vc, table


def test_verify_equals_sequential_decodes():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T, D, L = 2, 6, 3, 5, 16, 50
    kc, vc, table = _cache(rng, B, Hkv, L, D)
    q = rng.standard_normal((B, Hq, T, D))
    out, lse = verify_attention(q, kc, vc, table, np.full(B, L), 0.25)
    for t in range(T):
        o1, l1 = decode_attention(q[:, :, t], kc, vc, table, np.full(B, L - T + t + 1), 0.25)
        np.testing.assert_allclose(out[:, :, t], o1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, t], l1, rtol=1e-12)


def test_draft_full_set_equals_decode():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, L = 2, 8, 2, 16, 41
    kc, vc, table = _cache(rng, B, Hkv, L, D)
    q = rng.standard_normal((B, Hq, D))
    lens = np.array([L, L - 7])
    ref, ref_lse = decode_attention(q, kc, vc, table, lens, 0.3)
    # all rows through the index list, empty tail
    sel = np.tile(np.arange(L, dtype=np.int32), (B, Hkv, 1))
    o, l = draft_attention(q, kc, vc, table, lens, sel, lens, lens, 0.3)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, ref_lse, rtol=1e-12)
    # all rows through the dense tail, empty list
    o, l = draft_attention(q, kc, vc, table, lens, sel, np.zeros(B, int), np.zeros(B, int), 0.3)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)
    # a budget larger than the context (list + tail cover everything)
    o, l = draft_attention(q, kc, vc, table, lens, sel, np.array([10, 10]), np.array([10, 10]), 0.3)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)


def test_draft_set_is_order_free_and_filters_out_of_range():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, D, L = 1, 4, 1, 8, 30
    kc, vc, table = _cache(rng, B, Hkv, L, D)
    q = rng.standard_normal((B, Hq, D))
    sel = np.array([[[1, 4, 9, 17]]], dtype=np.int32)
    o1, _ = draft_attention(q, kc, vc, table, [L], sel, [4], [25], 0.3)
    o2, _ = draft_attention(q, kc, vc, table, [L], sel[:, :, ::-1].copy(), [4], [25], 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-13)
    # entries at or past the tail start and negative entries are not attended
    bad = np.array([[[1, 4, 9, 17, 26, -3]]], dtype=np.int32)
    o3, _ = draft_attention(q, kc, vc, table, [L], bad, [6], [25], 0.3)
    np.testing.assert_allclose(o1, o3, rtol=1e-13)
    assert list(draft_positions(L, bad[0, 0], 6, 25)) == [1, 4, 9, 17, 25, 26, 27, 28, 29]


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(17)
    n, D = 57, 12
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    ref, ref_lse = attend(q[None], K, V, 0.2)
    cuts = np.sort(rng.choice(np.arange(1, n), size=4, replace=False))
    parts = np.split(rng.permutation(n), cuts)
    parts.append(np.array([], dtype=int))          # an empty split contributes nothing
    ms, ls, os_ = zip(*[softmax_partial(q, K[p], V[p], 0.2) for p in parts])
    o, lse = merge_partials(ms, ls, os_)
    np.testing.assert_allclose(o, ref[0], rtol=1e-12, atol=1e-14)
    assert abs(lse - ref_lse[0]) < 1e-12


def test_degenerate_lengths():
    rng = np.random.default_rng(19)
    B, Hq, Hkv, T, D = 2, 4, 2, 4, 8
    kc, vc, table = _cache(rng, B, Hkv, 20, D)
    q = rng.standard_normal((B, Hq, T, D))
    out, lse = verify_attention(q, kc, vc, table, np.array([0, 2]), 0.3)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    # L = 2 < T = 4: queries 0, 1 see nothing; query 2 sees row 0; query 3 sees rows 0..1
    assert np.all(out[1, :, :2] == 0) and np.all(np.isneginf(lse[1, :, :2]))
    np.testing.assert_allclose(out[1, 0, 2], as_f64(vc[table[1, 0], 0, 0]), rtol=1e-14)
    o, l = decode_attention(q[:, :, 0], kc, vc, table, np.array([0, 0]), 0.3)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_bf16_bits_widen_exactly():
    vals = np.array([1.0, -2.5, 3.140625, 1e-3, -65504.0], dtype=np.float32)
    t = torch.from_numpy(vals).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(as_f64(bits), t.to(torch.float64).numpy())
