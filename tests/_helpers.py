"""Shared test helpers: tolerances, error metrics and oracle sub-cache extraction."""

import numpy as np
import torch

from kv_sparse_speculative_amd.synth import to_numpy

# Attention tolerance: per output row, max-abs error relative to the row's max-abs value
# (2e-3, the bound for fp32-accumulated outputs of bf16 attention).
ATTN_RTOL = 2e-3


def row_rel_err(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows are the last axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max(axis=-1)
    num = np.abs(got - ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0


def lse_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):          # -inf - (-inf) is masked out just below
        d = np.where(both_inf, 0.0, np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))
    return float(d.max()) if d.size else 0.0


def subcache(ns, seqs, lens=None):
    """Host copies of the cache blocks of sequences `seqs`, with a remapped block table.

    Returns (k, v, table, kv_lens_selected) for the oracle, covering only those sequences.
    """
    table = ns.block_table_np
    rows = []
    new_table = np.full((len(seqs), table.shape[1]), -1, dtype=np.int32)
    nxt = 0
    for i, b in enumerate(seqs):
        blocks = table[b][table[b] >= 0]
        rows.extend(blocks.tolist())
        new_table[i, : len(blocks)] = np.arange(nxt, nxt + len(blocks))
        nxt += len(blocks)
    idx = torch.as_tensor(rows, dtype=torch.long, device=ns.k_cache.device)
    k = to_numpy(ns.k_cache.index_select(0, idx))
    v = to_numpy(ns.v_cache.index_select(0, idx))
    return k, v, new_table


def host(t):
    return to_numpy(t)
