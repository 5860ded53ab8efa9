"""Attention over the KV cache: verify, decode and sparse draft (oracle, test infrastructure).

Follows MagicDec (arXiv 2408.11049v5):
  * Section 3.1: the target verifies gamma speculated tokens in one pass whose cost is
    T_V(B, S, gamma); together with the token being decoded that is gamma + 1 query tokens
    per sequence, each attending causally to the full KV cache.
  * Section 3.2: verification and plain decoding read the same KV cache, so decode is the
    one-query special case.
  * Section 4.1, Eq. (3): the draft decodes against a sparse KV subset of budget K
    (cost T_D(B, K)); Appendix A.1 (Fig. 8): for self-speculation that subset is drawn from
    the target's own cache.
  * Section 3.2 (last paragraph): grouped-query attention; q-head h reads KV head h // G
    with G = num_q_heads / num_kv_heads (the plain reading of a grouped layout).

The paper does not print the attention formula. Attention is exact, so this is its plain
definition: s_j = scale * <q, k_j>, a = softmax(s) over the attended set J,
o = sum_j a_j v_j, lse = log sum_j exp(s_j). The scale is 1/sqrt(head_dim) unless the
caller passes another (the paper is silent; this is the usual choice). An empty attended set
yields o = 0 and lse = -inf, which is also what merging zero partials gives.
"""

import numpy as np

from .kvcache import as_f64, gather_prefix, gather_rows


def attend(q_rows, keys, values, scale, limits=None):
    """Softmax attention of R query rows over n key/value rows, in float64.

    q_rows [R, D], keys [n, D], values [n, D]. If `limits` is given, row r attends only to
    key rows with index <= limits[r] (a causal bound); otherwise to all n rows.
    Returns (o [R, D], lse [R]).
    """
    q_rows = as_f64(q_rows)
    keys = as_f64(keys)
    values = as_f64(values)
    R, D = q_rows.shape
    n = keys.shape[0]
    out = np.zeros((R, D))
    lse = np.full(R, -np.inf)
    if n == 0:
        return out, lse
    s = scale * (q_rows @ keys.T)                      # [R, n]
    if limits is not None:
        limits = np.asarray(limits, dtype=np.int64)
        visible = np.arange(n)[None, :] <= limits[:, None]
        s = np.where(visible, s, -np.inf)
    for r in range(R):
        row = s[r]
        if not np.isfinite(row).any():
            continue
        m = row.max()
        e = np.exp(row - m)
        z = e.sum()
        out[r] = (e @ values) / z
        lse[r] = m + np.log(z)
    return out, lse


def _groups(num_q_heads, num_kv_heads):
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return num_q_heads // num_kv_heads


def _pairs(B, Hkv, pairs):
    if pairs is None:
        return [(b, g) for b in range(B) for g in range(Hkv)]
    return [(int(b), int(g)) for b, g in pairs]


def verify_attention(q, k_cache, v_cache, block_table, kv_lens, scale, pairs=None):
    """Causal attention of T = gamma + 1 query tokens per sequence over the full cache.

    q [B, Hq, T, D]. The cache of sequence b holds L_b = kv_lens[b] rows, the T new rows
    already written, so query t sits at position L_b - T + t and attends to [0, L_b - T + t].
    Returns (out [B, Hq, T, D], lse [B, Hq, T]); (b, g) pairs not listed in `pairs` are NaN.
    """
    B, Hq, T, D = q.shape
    Hkv = k_cache.shape[1]
    G = _groups(Hq, Hkv)
    out = np.full((B, Hq, T, D), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    for b, g in _pairs(B, Hkv, pairs):
        L = int(kv_lens[b])
        K = gather_prefix(k_cache, block_table, b, g, L)
        V = gather_prefix(v_cache, block_table, b, g, L)
        heads = list(range(g * G, (g + 1) * G))
        rows = as_f64(q[b, heads]).reshape(G * T, D)
        limits = np.tile(L - T + np.arange(T), G)
        o, l = attend(rows, K, V, scale, limits)
        out[b, heads] = o.reshape(G, T, D)
        lse[b, heads] = l.reshape(G, T)
    return out, lse


def decode_attention(q, k_cache, v_cache, block_table, kv_lens, scale, pairs=None):
    """One query per sequence over every cached row [0, L_b). q [B, Hq, D]."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _groups(Hq, Hkv)
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b, g in _pairs(B, Hkv, pairs):
        L = int(kv_lens[b])
        K = gather_prefix(k_cache, block_table, b, g, L)
        V = gather_prefix(v_cache, block_table, b, g, L)
        heads = list(range(g * G, (g + 1) * G))
        o, l = attend(as_f64(q[b, heads]), K, V, scale)
        out[b, heads] = o
        lse[b, heads] = l
    return out, lse


def draft_positions(kv_len, sel_row, sel_count, tail_lo):
    """The attended positions of a sparse draft query, in the order they are given.

    The set is the selected list sel_row[0:sel_count] followed by the dense tail
    [tail_lo, L). List entries outside [0, min(tail_lo, L)) are not attended (the list is
    meant to hold positions before the tail, ascending).
    """
    L = int(kv_len)
    lo = max(int(tail_lo), 0)
    sel = np.asarray(sel_row[: max(int(sel_count), 0)], dtype=np.int64)
    sel = sel[(sel >= 0) & (sel < min(lo, L))]
    tail = np.arange(lo, L, dtype=np.int64)
    return np.concatenate([sel, tail])


def draft_attention(q, k_cache, v_cache, block_table, kv_lens, sel_idx, sel_count, tail_lo,
                    scale, pairs=None):
    """One draft query per sequence over a sparse subset of the target's cache.

    q [B, Hq, D]; sel_idx int [B, Hkv, k_max]; sel_count, tail_lo, kv_lens int [B].
    Head h of group g attends to draft_positions(L_b, sel_idx[b, g], sel_count[b],
    tail_lo[b]). Returns (out [B, Hq, D], lse [B, Hq]).
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _groups(Hq, Hkv)
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b, g in _pairs(B, Hkv, pairs):
        pos = draft_positions(kv_lens[b], sel_idx[b, g], sel_count[b], tail_lo[b])
        K = gather_rows(k_cache, block_table, b, g, pos)
        V = gather_rows(v_cache, block_table, b, g, pos)
        heads = list(range(g * G, (g + 1) * G))
        o, l = attend(as_f64(q[b, heads]), K, V, scale)
        out[b, heads] = o
        lse[b, heads] = l
    return out, lse


def merge_partials(ms, ls, os_):
    """Combine softmax partials over disjoint key subsets into one result.

    Each partial s carries its own max m_s, normaliser l_s = sum exp(s - m_s) and
    unnormalised output o_s = sum exp(s - m_s) v. With M = max m_s and weights
    w_s = exp(m_s - M): o = sum w_s o_s / sum w_s l_s and lse = M + log sum w_s l_s.
    Partials with l_s = 0 (empty subsets, m_s = -inf) contribute nothing.
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    os_ = np.asarray(os_, dtype=np.float64)
    if not np.isfinite(ms).any():
        return np.zeros(os_.shape[1:]), -np.inf
    M = ms.max()
    w = np.where(np.isfinite(ms), np.exp(ms - M), 0.0)
    lam = (w * ls).sum()
    return (w[:, None] * os_).sum(axis=0) / lam, M + np.log(lam)


def softmax_partial(q_row, keys, values, scale):
    """The (m, l, o) partial of one query row over a key subset (see merge_partials)."""
    keys = as_f64(keys)
    values = as_f64(values)
    if keys.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(values.shape[1])
    s = scale * (keys @ as_f64(q_row))
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ values
