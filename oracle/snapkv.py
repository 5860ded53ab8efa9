"""SnapKV draft KV selection (oracle, test infrastructure).

MagicDec uses SnapKV as its static KV selection for self-speculation: Section 4.4 classes it
as static (the sparse cache is gathered once, with no per-query search), Section 5.2 reports
2049 as its best draft budget, Table 2 runs it at 64k-100k prefill, and Appendix A.1 (Fig. 8)
states that the static compressed cache is produced during prefill and then used for
drafting. The paper does not print SnapKV's steps. The reading taken here (observation-window
voting, pooling, per-head top-k):

  1. For every q-head h of KV group g and every observation query i in [0, w), sitting at
     prompt position P - w + i, take its full causal softmax over keys [0, P - w + i].
  2. Column score c_g[j] = sum over h in g and i < w of those probabilities, for the
     candidate positions j in [0, P - w) (the window itself is always kept). Summing and
     averaging give the same selection, so the sum is used.
  3. pooled_g[j] = max of c_g over the centred window |j' - j| <= (pool - 1) / 2, clipped to
     [0, P - w) (positions outside contribute nothing).
  4. Keep k = budget - w candidates: all of them when P - w <= k, else the k largest pooled
     scores, ties going to the lower position; report them ascending.
  5. The draft then attends to the kept positions plus the dense tail [P - w, L): the
     observation window and every later token.
"""

import numpy as np

from .kvcache import as_f64, gather_prefix


def snapkv_scores(q_obs, k_cache, block_table, prompt_lens, w, scale, pairs=None):
    """Column scores c [B, Hkv, max_b(P_b - w)] (step 2); entries past P_b - w are NaN.

    q_obs [B, Hq, w, D] holds the observation-window queries of each prompt.
    """
    B, Hq, w_, D = q_obs.shape
    if w_ != w:
        raise ValueError("q_obs window length does not match w")
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    prompt_lens = np.asarray(prompt_lens, dtype=np.int64)
    n_max = max(int(prompt_lens.max()) - w, 0)
    c = np.full((B, Hkv, n_max), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in pairs:
        P = int(prompt_lens[b])
        n = max(P - w, 0)
        K = gather_prefix(k_cache, block_table, b, g, P)
        col = np.zeros(n)
        for h in range(g * G, (g + 1) * G):
            q = as_f64(q_obs[b, h])                      # [w, D]
            s = scale * (q @ K.T)                        # [w, P]
            for i in range(w):
                last = P - w + i                         # causal bound of query i
                if last < 0:
                    continue
                row = s[i, : last + 1]
                e = np.exp(row - row.max())
                a = e / e.sum()
                col += a[:n]
        c[b, g, :n] = col
    return c


def max_pool(scores, pool):
    """Centred same-length 1-D max-pool (step 3); out-of-range neighbours are ignored."""
    if pool % 2 != 1:
        raise ValueError("pool kernel must be odd")
    r = (pool - 1) // 2
    n = scores.shape[0]
    out = np.empty(n)
    for j in range(n):
        out[j] = scores[max(0, j - r): min(n, j + r + 1)].max()
    return out


def top_k_positions(pooled, k):
    """Step 4: the k largest values (ties to the lower position), returned ascending."""
    n = pooled.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = sorted(range(n), key=lambda j: (-pooled[j], j))
    return np.sort(np.asarray(order[:k], dtype=np.int64))


def select_from_scores(scores, prompt_lens, w, pool, budget):
    """Steps 3-4 on given column scores [B, Hkv, >= P_b - w].

    Returns (sel_idx int32 [B, Hkv, budget - w] padded with -1, sel_count int32 [B]).
    """
    B, Hkv = scores.shape[:2]
    k = budget - w
    sel_idx = np.full((B, Hkv, k), -1, dtype=np.int32)
    sel_count = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = max(int(prompt_lens[b]) - w, 0)
        sel_count[b] = min(k, n)
        for g in range(Hkv):
            keep = top_k_positions(max_pool(np.asarray(scores[b, g, :n], dtype=np.float64), pool), k)
            sel_idx[b, g, : keep.shape[0]] = keep
    return sel_idx, sel_count


def snapkv_select(q_obs, k_cache, block_table, prompt_lens, w, pool, budget, scale):
    """The whole selection: returns (sel_idx, sel_count, scores)."""
    if budget <= w:
        raise ValueError("budget must exceed the observation window")
    c = snapkv_scores(q_obs, k_cache, block_table, prompt_lens, w, scale)
    sel_idx, sel_count = select_from_scores(c, prompt_lens, w, pool, budget)
    return sel_idx, sel_count, c
