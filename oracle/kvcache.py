"""Exact input widening and paged KV-cache row addressing (oracle, test infrastructure).

The paper (MagicDec, Section 1 insight (1) and Section 3.2) identifies the per-layer KV
cache, which grows with batch size and context length, as the dominant memory and
bandwidth term; it does not fix a memory layout. The reading taken here: one paged layout
for every workload. A cache tensor has shape [num_blocks, num_kv_heads, block_size,
head_dim]; logical row j of sequence b and KV head g lives in physical block
block_table[b, j // block_size] at offset j % block_size. Contiguous caches are the
special case of an identity block table.
"""

import numpy as np


def as_f64(x):
    """Widen stored values to float64 exactly.

    Arrays of dtype uint16 hold bfloat16 bit patterns (the upper half of an IEEE binary32);
    they are widened by placing the 16 bits in the high half of a 32-bit word. float32 and
    float64 arrays widen with a plain cast. No rounding happens on any path.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {x.dtype}")


def gather_rows(cache, block_table, b, g, positions):
    """Rows `positions` of sequence b, KV head g, as float64 [len(positions), head_dim].

    Positions are logical token indices; the block table maps them to physical blocks.
    """
    positions = np.asarray(positions, dtype=np.int64)
    bs = cache.shape[2]
    blocks = np.asarray(block_table)[b, positions // bs]
    return as_f64(cache[blocks, g, positions % bs, :])


def gather_prefix(cache, block_table, b, g, length):
    """Rows [0, length) of sequence b, KV head g, as float64 [length, head_dim]."""
    return gather_rows(cache, block_table, b, g, np.arange(int(length)))


def append_rows(k_cache, v_cache, block_table, k_new, v_new, start):
    """Write T new K/V rows per sequence into copies of the paged caches.

    MagicDec Section 3.1: the target scores gamma + 1 tokens per verify pass, and those
    tokens' keys and values become part of the cache the pass attends to; Appendix A.1
    (Fig. 8): the draft keeps its own compressed cache that grows the same way. The paper
    prints no append rule; the reading taken: row t of sequence b goes to logical position
    start[b] + t through the block table. A row whose position lies outside the table
    (negative, or >= max_blocks * block_size) or whose physical block id is outside
    [0, num_blocks) is not written.

    k_new, v_new: [B, num_kv_heads, T, head_dim] in the caches' stored dtype. Returns
    (k_cache', v_cache').
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    table = np.asarray(block_table)
    nb, hkv, bs, _ = k_out.shape
    B, H, T, _ = np.asarray(k_new).shape
    for b in range(B):
        for t in range(T):
            pos = int(start[b]) + t
            if pos < 0 or pos >= table.shape[1] * bs:
                continue
            blk = int(table[b, pos // bs])
            if not 0 <= blk < nb:
                continue
            for g in range(H):
                k_out[blk, g, pos % bs] = k_new[b, g, t]
                v_out[blk, g, pos % bs] = v_new[b, g, t]
    return k_out, v_out


def _nan_row(dtype, width):
    """A row of NaN in the stored dtype (bf16 bit pattern 0x7FC0 for uint16 storage)."""
    if np.dtype(dtype) == np.uint16:
        return np.full(width, 0x7FC0, dtype=np.uint16)
    return np.full(width, np.nan, dtype=dtype)


def compact_rows(cache, block_table, kv_lens, sel_idx, sel_count, tail_lo, max_tail=None):
    """The draft set of every (sequence, KV head) as one contiguous logical row list.

    MagicDec Appendix A.1 (Fig. 8): the static compressed KV is built once at prefill and the
    draft reads it. Reading: the compressed cache of (b, g) holds, in this order, the listed
    rows sel_idx[b, g, 0:n] (n = sel_count[b] clamped to [0, k_max]) and then the recent rows
    [tail_lo[b], kv_lens[b]), so a plain decode over it attends to exactly the draft set of
    draft_attention. A compressed cache holds one row per slot, so a listed position outside
    [0, tail_lo) (which the sparse draft would skip) cannot be left out; its slot holds a row
    of NaN, as does every slot of a sequence whose tail is longer than max_tail (its length
    is then cut to n + max_tail), so such inputs cannot pass unnoticed.

    Returns a list over b of arrays [num_kv_heads, n_b, head_dim] in the stored dtype (rows
    are copied, not widened) and the lengths n_b.
    """
    table = np.asarray(block_table)
    nb, hkv, bs, D = cache.shape
    k_max = sel_idx.shape[2]
    out, lens = [], []
    for b in range(len(kv_lens)):
        L = int(kv_lens[b])
        lo = min(max(int(tail_lo[b]), 0), L)
        n = min(max(int(sel_count[b]), 0), k_max)
        tail = L - lo
        poison = max_tail is not None and tail > max_tail
        if poison:
            tail = max_tail
        rows = np.empty((hkv, n + tail, D), dtype=cache.dtype)
        for g in range(hkv):
            pos = np.concatenate([np.asarray(sel_idx[b, g, :n], dtype=np.int64),
                                  np.arange(lo, lo + tail, dtype=np.int64)])
            for j, p in enumerate(pos):
                valid = (0 <= p < lo) if j < n else True
                blk = int(table[b, p // bs]) if valid else -1
                if poison or not valid or not 0 <= blk < nb:
                    rows[g, j] = _nan_row(cache.dtype, D)
                else:
                    rows[g, j] = cache[blk, g, p % bs]
        out.append(rows)
        lens.append(n + tail)
    return out, np.asarray(lens, dtype=np.int64)
