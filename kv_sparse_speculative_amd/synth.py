"""Seeded synthetic inputs for the attention, selection and acceptance calls.

This module draws inputs only; it holds none of the method's arithmetic, and both the HIP
library's tests and the CPU oracle's tests take their inputs from here. The stored bits are
the single source of truth: values are drawn in float32 and stored in the workload's dtype
(bfloat16 by round-to-nearest-even), and the oracle widens exactly those bits.

Recipe (per workload, seed = workload seed, one sub-seed per tensor):
  * prompt lengths P_b: fixed, or uniform integers in [lo, hi] for a ragged batch;
  * cache capacity per sequence: P_b + gamma + 1 rows (prompt + the verified tokens), in
    blocks of `block_size` rows; the block table is the identity or a seeded permutation of
    the block pool; unused table slots hold -1;
  * K, V, every query ~ N(0, 1);
  * planted keys: for a share `planted_frac` of the candidate positions [0, P_b - w) of every
    (sequence, KV head), distinct seeded positions get k = q_obs[h, i] + N(0, 0.1^2) for a
    seeded q-head h of the group and window query i (makes window attention peaky);
  * acceptance logits ~ N(0, 2) (standard deviation sqrt(2)), target and draft drawn
    independently; draft tokens uniform over the vocabulary; to exercise greedy acceptance a
    seeded prefix of n_b ~ U{0..gamma} draft tokens per sequence is planted as the target's
    clear winner (its target logit set to 20).
"""

import math
from types import SimpleNamespace

import numpy as np
import torch

from .workloads import Workload

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, gen, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def to_numpy(t):
    """A host numpy copy of a tensor; bfloat16 becomes its uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def prompt_lengths(wl: Workload, batch=None, prompt=None):
    """Seeded prompt lengths [B] (int64 numpy)."""
    B = batch or wl.batch
    lo, hi = prompt if prompt is not None else wl.prompt
    if lo == hi:
        return np.full(B, lo, dtype=np.int64)
    rng = np.random.default_rng(wl.seed * 100 + 1)
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


def generate(wl: Workload, device="cpu", batch=None, prompt=None, parts=("attn", "accept"),
             vocab=None):
    """Draw the inputs of one workload (optionally with a smaller batch / prompt range).

    Returns a namespace of torch tensors on `device` plus int metadata.
    """
    B = batch or wl.batch
    T = wl.gamma + 1
    dt = _TORCH_DTYPE[wl.dtype]
    ns = SimpleNamespace(workload=wl, batch=B, gamma=wl.gamma, T=T, device=device)
    P = prompt_lengths(wl, B, prompt)
    ns.prompt_lens_np = P
    cap = P + T
    bs = wl.block_size
    nblk = (cap + bs - 1) // bs
    total = int(nblk.sum())
    max_blocks = int(nblk.max())
    if wl.shuffled_blocks:
        perm = np.random.default_rng(wl.seed * 100 + 2).permutation(total).astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[start: start + nblk[b]]
        start += nblk[b]
    ns.block_table_np = table
    ns.num_blocks = total
    ns.max_blocks = max_blocks
    ns.block_table = torch.from_numpy(table).to(device)
    ns.prompt_lens = torch.from_numpy(P.astype(np.int32)).to(device)
    ns.kv_lens_verify = torch.from_numpy((P + T).astype(np.int32)).to(device)
    ns.kv_lens_draft = torch.from_numpy((P + 1).astype(np.int32)).to(device)
    ns.max_prompt = int(P.max())
    Hq, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim

    if "attn" in parts:
        gk = _gen(device, wl.seed * 100 + 10)
        gv = _gen(device, wl.seed * 100 + 11)
        ns.k_cache = _normal((total, Hkv, bs, D), gk, device).to(dt)
        ns.v_cache = _normal((total, Hkv, bs, D), gv, device).to(dt)
        gq = _gen(device, wl.seed * 100 + 12)
        ns.q_verify = _normal((B, Hq, T, D), gq, device).to(dt)
        ns.q_draft = _normal((B, Hq, D), gq, device).to(dt)
        if wl.snapkv is not None:
            budget, w, pool = wl.snapkv
            ns.q_obs = _normal((B, Hq, w, D), gq, device).to(dt)
            if wl.planted_frac > 0:
                _plant_keys(ns, wl, P, w, device)

    if "accept" in parts:
        V = vocab or wl.vocab
        ga = _gen(device, wl.seed * 100 + 20)
        ns.vocab = V
        ns.target_logits = _normal((B, T, V), ga, device, std=math.sqrt(2.0))
        ns.draft_logits = _normal((B, wl.gamma, V), ga, device, std=math.sqrt(2.0))
        rng = np.random.default_rng(wl.seed * 100 + 21)
        tokens = rng.integers(0, V, size=(B, wl.gamma)).astype(np.int32)
        ns.draft_tokens = torch.from_numpy(tokens).to(device)
        n_plant = rng.integers(0, wl.gamma + 1, size=B)
        for b in range(B):
            for i in range(int(n_plant[b])):
                ns.target_logits[b, i, int(tokens[b, i])] = 20.0
    return ns


def _plant_keys(ns, wl, P, w, device):
    """Overwrite a seeded share of candidate keys with noisy copies of window queries."""
    rng = np.random.default_rng(wl.seed * 100 + 30)
    gn = _gen(device, wl.seed * 100 + 31)
    G = wl.group
    bs = wl.block_size
    table = ns.block_table_np
    for b in range(ns.batch):
        n = int(P[b]) - w
        m = int(round(wl.planted_frac * n))
        if m <= 0:
            continue
        for g in range(wl.num_kv_heads):
            pos = rng.choice(n, size=m, replace=False)
            heads = g * G + rng.integers(0, G, size=m)
            qi = rng.integers(0, w, size=m)
            src = ns.q_obs[b, torch.from_numpy(heads).to(device),
                           torch.from_numpy(qi).to(device)].float()
            rows = src + _normal(src.shape, gn, device, std=0.1)
            blk = torch.from_numpy(table[b, pos // bs].astype(np.int64)).to(device)
            off = torch.from_numpy((pos % bs).astype(np.int64)).to(device)
            ns.k_cache[blk, g, off] = rows.to(ns.k_cache.dtype)
