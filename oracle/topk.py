"""Dynamic Top-K draft attention (oracle, test infrastructure).

MagicDec names TopK attention as the dynamic selection with the highest acceptance rate
(Fig. 1(c)) whose per-query search the paper judges too costly for selection (Section 4.4,
Static vs Dynamic): unlike StreamingLLM or SnapKV, the subset is chosen anew for every draft
query, so T_select(B, S, K) is paid on every draft step and grows with B * S. The paper gives
no formula. Readings taken here:

  * The subset is chosen per KV head, shared by the G query heads of the group (they read one
    KV subset, as in the draft of Section 4.1). A key's score is the sum over those G heads of
    its softmax probability under the current draft query; for G = 1 this ranks keys by the
    raw score q . k, which is exact top-k attention.
  * The current token (position L - 1) is always attended; the k kept keys come from
    [0, L - 1), ties to the lower position, reported ascending.

That is the SnapKV rule of oracle.snapkv with the draft query as a one-token observation
window (w = 1) and no pooling (pool = 1), so this module composes those functions.
"""

import numpy as np

from .attention import draft_attention
from .snapkv import snapkv_select


def topk_positions(q, k_cache, block_table, kv_lens, k, scale):
    """q [B, Hq, D] at positions L_b - 1 -> (sel_idx [B, Hkv, k], sel_count [B], scores)."""
    q_obs = np.asarray(q)[:, :, None, :]
    return snapkv_select(q_obs, k_cache, block_table, np.asarray(kv_lens), 1, 1, k + 1, scale)


def topk_draft_attention(q, k_cache, v_cache, block_table, kv_lens, k, scale):
    """One draft query per sequence over its dynamic top-k keys plus itself.

    Returns (out [B, Hq, D], lse [B, Hq], sel_idx, sel_count)."""
    sel, cnt, _ = topk_positions(q, k_cache, block_table, kv_lens, k, scale)
    L = np.asarray(kv_lens, dtype=np.int64)
    out, lse = draft_attention(q, k_cache, v_cache, block_table, L, sel, cnt,
                               np.maximum(L - 1, 0), scale)
    return out, lse, sel, cnt
