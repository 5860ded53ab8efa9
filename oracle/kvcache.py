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
