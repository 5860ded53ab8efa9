"""Pins of the oracle's cache maintenance (KV append, compact draft cache) against things other
than itself: the logical view of a paged cache, untouched physical blocks, and the identity
that a plain decode over the compact rows is the sparse draft over the original cache."""

import numpy as np
import pytest

from oracle.attention import decode_attention, draft_attention, verify_attention
from oracle.kvcache import append_rows, compact_rows, gather_prefix, gather_rows

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _paged_cache(rng, B, Hkv, max_blocks, bs, D, spare=3, dtype=np.float32):
    """Random paged caches with a shuffled table; `spare` physical blocks belong to nobody."""
    nb = B * max_blocks + spare
    perm = rng.permutation(nb)
    table = perm[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    k = rng.standard_normal((nb, Hkv, bs, D)).astype(dtype)
    v = rng.standard_normal((nb, Hkv, bs, D)).astype(dtype)
    return k, v, table, perm[B * max_blocks:]


def test_append_lands_at_logical_positions():
    rng = np.random.default_rng(11)
    B, Hkv, mb, bs, D, T = 3, 2, 4, 4, 8, 3
    k, v, table, _ = _paged_cache(rng, B, Hkv, mb, bs, D)
    start = np.array([0, 5, 13])                      # spans block boundaries
    kn = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    k2, v2, = append_rows(k, v, table, kn, vn, start)
    for b in range(B):
        for g in range(Hkv):
            pos = start[b] + np.arange(T)
            np.testing.assert_array_equal(gather_rows(k2, table, b, g, pos), kn[b, g].astype(np.float64))
            np.testing.assert_array_equal(gather_rows(v2, table, b, g, pos), vn[b, g].astype(np.float64))
            # every other logical row of the sequence is unchanged
            other = np.setdiff1d(np.arange(mb * bs), pos)
            np.testing.assert_array_equal(gather_rows(k2, table, b, g, other),
                                          gather_rows(k, table, b, g, other))


def test_append_leaves_foreign_blocks_and_skips_out_of_range():
    rng = np.random.default_rng(12)
    B, Hkv, mb, bs, D, T = 2, 2, 3, 4, 4, 4
    k, v, table, spare = _paged_cache(rng, B, Hkv, mb, bs, D)
    kn = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    # sequence 0 starts 2 rows before the end of its table: rows 2 and 3 fall outside;
    # sequence 1 starts at -2: rows 0 and 1 fall outside
    start = np.array([mb * bs - 2, -2])
    k2, v2 = append_rows(k, v, table, kn, kn, start)
    np.testing.assert_array_equal(k2[spare], k[spare])
    np.testing.assert_array_equal(gather_rows(k2, table, 0, 1, [mb * bs - 2, mb * bs - 1]),
                                  kn[0, 1, :2].astype(np.float64))
    np.testing.assert_array_equal(gather_rows(k2, table, 1, 0, [0, 1]), kn[1, 0, 2:].astype(np.float64))
    changed = np.argwhere((k2 != k).any(axis=(1, 2, 3))).ravel()
    assert set(changed) <= {int(table[0, mb - 1]), int(table[1, 0])}
    # a block id outside the cache is not written
    bad = table.copy()
    bad[0, 0] = k.shape[0] + 7
    k3, _ = append_rows(k, v, bad, kn, kn, np.array([0, 0]))
    np.testing.assert_array_equal(k3[table[0, 0]], k[table[0, 0]])


def test_append_then_verify_equals_attention_over_the_extended_sequence():
    """Writing the gamma + 1 verify rows and attending equals attending over the logical
    prefix with those rows concatenated (the verify pass sees its own tokens)."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, mb, bs, D, T = 2, 4, 2, 6, 4, 8, 3
    k, v, table, _ = _paged_cache(rng, B, Hkv, mb, bs, D, dtype=np.float64)
    L0 = np.array([9, 17])
    kn = rng.standard_normal((B, Hkv, T, D))
    vn = rng.standard_normal((B, Hkv, T, D))
    k2, v2 = append_rows(k, v, table, kn, vn, L0)
    q = rng.standard_normal((B, Hq, T, D))
    out, lse = verify_attention(q, k2, v2, table, L0 + T, 0.3)
    # the same logical rows in a contiguous cache with an identity table
    cap = mb * bs
    kc = np.zeros((B * mb, Hkv, bs, D))
    vc = np.zeros((B * mb, Hkv, bs, D))
    ident = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    for b in range(B):
        for g in range(Hkv):
            rows_k = np.concatenate([gather_prefix(k, table, b, g, L0[b]), kn[b, g]])
            rows_v = np.concatenate([gather_prefix(v, table, b, g, L0[b]), vn[b, g]])
            for j in range(rows_k.shape[0]):
                kc[ident[b, j // bs], g, j % bs] = rows_k[j]
                vc[ident[b, j // bs], g, j % bs] = rows_v[j]
    assert cap >= L0.max() + T
    out2, lse2 = verify_attention(q, kc, vc, ident, L0 + T, 0.3)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n_list", [0, 5, 11])
def test_decode_over_compact_rows_is_the_sparse_draft(n_list):
    rng = np.random.default_rng(20 + n_list)
    B, Hq, Hkv, mb, bs, D = 3, 6, 2, 8, 4, 16
    k, v, table, _ = _paged_cache(rng, B, Hkv, mb, bs, D, dtype=np.float64)
    L = np.array([20, 31, 26])
    tail_lo = np.array([14, 25, 26])                   # the last sequence has an empty tail
    k_max = 12
    sel = np.full((B, Hkv, k_max), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            sel[b, g, :n_list] = np.sort(rng.choice(tail_lo[b], size=n_list, replace=False))
    cnt = np.full(B, n_list)
    q = rng.standard_normal((B, Hq, D))
    ref, ref_lse = draft_attention(q, k, v, table, L, sel, cnt, tail_lo, 0.25)

    krows, lens = compact_rows(k, table, L, sel, cnt, tail_lo)
    vrows, lens_v = compact_rows(v, table, L, sel, cnt, tail_lo)
    np.testing.assert_array_equal(lens, cnt + L - tail_lo)
    np.testing.assert_array_equal(lens, lens_v)
    # lay the compact rows into their own contiguous cache and decode over it
    cb = (int(lens.max()) + bs - 1) // bs
    kc = np.zeros((B * cb, Hkv, bs, D))
    vc = np.zeros((B * cb, Hkv, bs, D))
    ident = np.arange(B * cb, dtype=np.int32).reshape(B, cb)
    for b in range(B):
        for j in range(int(lens[b])):
            kc[ident[b, j // bs], :, j % bs] = krows[b][:, j]
            vc[ident[b, j // bs], :, j % bs] = vrows[b][:, j]
    out, lse = decode_attention(q, kc, vc, ident, lens, 0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_compact_rows_copy_stored_bits():
    """bf16 rows are copied as stored bit patterns, listed rows first in list order."""
    rng = np.random.default_rng(30)
    B, Hkv, mb, bs, D = 1, 2, 3, 4, 8
    k = rng.integers(0, 1 << 16, size=(B * mb, Hkv, bs, D), dtype=np.uint16)
    table = np.array([[2, 0, 1]], dtype=np.int32)
    sel = np.array([[[3, 1, -1], [0, 7, -1]]], dtype=np.int32)
    rows, lens = compact_rows(k, table, np.array([12]), sel, np.array([2]), np.array([9]))
    assert rows[0].dtype == np.uint16 and lens[0] == 2 + 3
    expect_pos = [[3, 1, 9, 10, 11], [0, 7, 9, 10, 11]]
    for g in range(Hkv):
        for j, p in enumerate(expect_pos[g]):
            np.testing.assert_array_equal(rows[0][g, j], k[table[0, p // bs], g, p % bs])


def test_compact_rows_poison_invalid_inputs():
    """Listed positions outside [0, tail_lo), bad block ids and over-long tails give NaN rows."""
    rng = np.random.default_rng(31)
    B, Hkv, mb, bs, D = 2, 1, 4, 4, 4
    k = rng.standard_normal((B * mb, Hkv, bs, D)).astype(np.float32)
    table = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    table[1, 0] = 99                                       # rows 0..3 of sequence 1 unreadable
    sel = np.array([[[2, 12, -1]], [[1, 5, 6]]], dtype=np.int32)
    rows, lens = compact_rows(k, table, np.array([14, 10]), sel, np.array([2, 5]),
                              np.array([10, 8]), max_tail=4)
    np.testing.assert_array_equal(lens, [2 + 4, 3 + 2])    # sel_count clamps to k_max = 3
    assert not np.isnan(rows[0][0, 0]).any()               # position 2: fine
    assert np.isnan(rows[0][0, 1]).all()                   # 12 >= tail_lo: poisoned
    assert np.isnan(rows[1][0, 0]).all()                   # block id 99
    assert not np.isnan(rows[1][0, 1:]).any()
    rows, lens = compact_rows(k, table, np.array([14, 10]), sel, np.array([2, 0]),
                              np.array([10, 2]), max_tail=3)
    assert lens[1] == 3 and np.isnan(rows[1]).all()       # tail 8 > max_tail 3
