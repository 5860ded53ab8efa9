"""StreamingLLM draft KV set: attention sinks plus a recent window (oracle, test infrastructure).

MagicDec Section 5.1 (Setup) drafts with a StreamingLLM-style sparse KV and Table 1 uses a
draft budget of 512; Section 5.2 finds 512 the best StreamingLLM budget. The paper names the
method (sink tokens plus recent window) without giving its index arithmetic. The reading
taken here: with L cached rows, the draft attends to the first `sink` rows and the most
recent `window` rows, S = [0, min(sink, L)) U [max(sink, L - window), L); the current token's
own row is inside the window, so |S| = sink + window once L >= sink + window, and S = [0, L)
below that. Keys keep their original positions (no re-rotation): self-speculation reuses the
target's own cache (Appendix A.1, Fig. 8).
"""

import numpy as np


def streaming_positions(kv_len, sink, window):
    """The StreamingLLM set of a sequence with kv_len cached rows, ascending."""
    L = int(kv_len)
    head = np.arange(0, min(sink, L), dtype=np.int64)
    tail = np.arange(max(sink, L - window), L, dtype=np.int64)
    return np.concatenate([head, tail])


def streaming_set(kv_lens, num_kv_heads, sink, window):
    """The set in the sparse-draft encoding: selected list + dense tail.

    Returns (sel_idx int32 [B, Hkv, sink], sel_count int32 [B], tail_lo int32 [B]):
    the list holds the sink rows [0, min(sink, L)) (padded with -1), and the tail starts at
    max(sink, L - window). All KV heads share the same set.
    """
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    B = kv_lens.shape[0]
    sel_idx = np.full((B, num_kv_heads, sink), -1, dtype=np.int32)
    sel_count = np.zeros(B, dtype=np.int32)
    tail_lo = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(kv_lens[b])
        n = min(sink, L)
        sel_idx[b, :, :n] = np.arange(n, dtype=np.int32)
        sel_count[b] = n
        tail_lo[b] = max(sink, L - window)
    return sel_idx, sel_count, tail_lo
