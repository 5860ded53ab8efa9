"""GPU parity of the draft-token sampler (draft_sample) against the oracle: greedy tokens
bit-exact; sampled tokens identical except where the oracle's two best race keys are within
1e-5 (a near-tie that float32 may order differently)."""

import numpy as np
import pytest
import torch

import oracle.accept as oacc
from oracle.philox import draft_uniforms
from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

from _helpers import host

pytestmark = pytest.mark.gpu


def _near_tie(z, t, seed, offset, b, step):
    """True if the oracle's race over softmax(z / t) has its top two keys within 1e-5."""
    p = oacc.softmax(z, t)
    u = draft_uniforms(seed, offset, b, step, z.shape[0])
    keys = np.where(p > 0, -np.log(u) / np.where(p > 0, p, 1.0), np.inf)
    a, c = np.partition(keys, 1)[:2]
    return (c - a) <= 1e-5 * a


@pytest.mark.parametrize("name,batch,vocab", [("tiny_fp32", 2, None), ("llama8b_ctx8k", 16, None),
                                              ("qwen32b_ragged", 8, None),
                                              ("llama8b_ctx8k", 64, 3000)])
@pytest.mark.parametrize("temp", [0.0, 0.7, 1.0])
def test_draft_sample_matches_oracle(name, batch, vocab, temp):
    ns = generate(WORKLOADS[name], device="cuda", batch=batch, parts=("accept",), vocab=vocab)
    logits = ns.draft_logits[:, 0].contiguous()
    seed, offset, step = 0xD7AF7 + batch, 5, 2
    tok, st = kvss.draft_sample(logits, temp, seed, offset, step, want_stats=True)
    torch.cuda.synchronize()
    z = host(logits).astype(np.float64)
    ref = oacc.draft_sample(z, temp, seed, offset, step)
    g = host(tok)
    # the statistics row: argmax bit-exact, max within float32 rounding
    np.testing.assert_array_equal(host(st)[:, 3].astype(np.int64),
                                  [oacc.argmax_lowest(r) for r in z])
    if temp == 0:
        np.testing.assert_array_equal(g, ref)
        assert (host(st)[:, :3] == 0).all()        # greedy: only the argmax is written
        return
    np.testing.assert_allclose(host(st)[:, 0], z.max(axis=1) / temp, rtol=1e-6)
    # sum of exp(z / t - max): float32 terms summed over the row, relative error << 1e-4
    y = z / temp
    ref_s = np.exp(y - y.max(axis=1, keepdims=True)).sum(axis=1)
    np.testing.assert_allclose(host(st)[:, 1], ref_s, rtol=1e-4)
    assert (host(st)[:, 2] == 0).all()
    bad = [b for b in range(batch) if g[b] != ref[b] and not _near_tie(z[b], temp, seed, offset, b, step)]
    near = sum(1 for b in range(batch) if g[b] != ref[b]) - len(bad)
    print(f"draft sample {name} V={z.shape[1]} t={temp}: near-tie flips {near}")
    assert not bad, bad


def test_draft_sample_step_and_stream_change_the_draw():
    """Different steps draw different uniforms; the draft stream is not the acceptance race's."""
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", batch=64, parts=("accept",), vocab=500)
    logits = (ns.draft_logits[:, 0] * 0.0).contiguous()          # uniform law: tokens = race winners
    a, _ = kvss.draft_sample(logits, 1.0, 11, 3, 0)
    b, _ = kvss.draft_sample(logits, 1.0, 11, 3, 1)
    target = logits[:, None, :].contiguous()
    c, _, _ = kvss.spec_accept(target, None, torch.empty((64, 0), dtype=torch.int32, device="cuda"),
                               1.0, 11, 3)
    torch.cuda.synchronize()
    assert (host(a) != host(b)).mean() > 0.9
    assert (host(a) != host(c)[:, 0]).mean() > 0.9


@pytest.mark.parametrize("vocab,shift", [(1001, 0), (4096, 1), (9000, 3)],
                         ids=["ragged_vocab", "unaligned_rows", "ragged_two_slices"])
@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_draft_sample_scalar_path(vocab, shift, temp):
    """Rows that are not whole 16-byte blocks (vocab % 4 != 0, or a base 4 bytes past 16-byte
    alignment) take the element-wise path; tokens and statistics still match the oracle."""
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", batch=9, parts=("accept",), vocab=vocab)
    src = ns.draft_logits[:, 0].contiguous()
    buf = torch.empty(src.numel() + 4, dtype=torch.float32, device="cuda")
    logits = buf[shift:shift + src.numel()].view(src.shape)
    logits.copy_(src)
    seed, offset, step = 123, 7, 3
    tok, st = kvss.draft_sample(logits, temp, seed, offset, step, want_stats=True)
    torch.cuda.synchronize()
    z = host(src).astype(np.float64)
    ref = oacc.draft_sample(z, temp, seed, offset, step)
    g = host(tok)
    np.testing.assert_array_equal(host(st)[:, 3].astype(np.int64), [oacc.argmax_lowest(r) for r in z])
    if temp == 0:
        np.testing.assert_array_equal(g, ref)
        assert (host(st)[:, :3] == 0).all()        # greedy: only the argmax is written
        return
    ref_s = np.exp(z / temp - (z / temp).max(axis=1, keepdims=True)).sum(axis=1)
    np.testing.assert_allclose(host(st)[:, 1], ref_s, rtol=1e-4)
    bad = [b for b in range(9) if g[b] != ref[b] and not _near_tie(z[b], temp, seed, offset, b, step)]
    assert not bad, bad


@pytest.mark.parametrize("temp", [1e-3, 1e4], ids=["cold", "hot"])
def test_draft_sample_extreme_temperatures(temp):
    """A cold temperature concentrates the law on the argmax (z/t spans ~1e4 in log space); a hot
    one makes it nearly uniform. Tokens match the oracle except at flagged near-ties, and the
    row statistics stay finite."""
    ns = generate(WORKLOADS["llama8b_ctx8k"], device="cuda", batch=16, parts=("accept",), vocab=5000)
    logits = ns.draft_logits[:, 0].contiguous()
    seed, offset, step = 99, 1, 0
    tok, st = kvss.draft_sample(logits, temp, seed, offset, step, want_stats=True)
    torch.cuda.synchronize()
    z = host(logits).astype(np.float64)
    ref = oacc.draft_sample(z, temp, seed, offset, step)
    g = host(tok)
    assert np.isfinite(host(st)).all()
    y = z / temp
    ref_s = np.exp(y - y.max(axis=1, keepdims=True)).sum(axis=1)
    np.testing.assert_allclose(host(st)[:, 1], ref_s, rtol=1e-4)
    bad = [b for b in range(16) if g[b] != ref[b] and not _near_tie(z[b], temp, seed, offset, b, step)]
    assert not bad, bad
