"""GPU statistical check of spec_accept's sampling law against closed forms (no oracle run):
2^20 speculative rounds on a vocabulary of 8 with gamma = 3, draft tokens drawn from q.

Speculative sampling (Leviathan et al., the rule MagicDec Section 3.1 uses) must give:
  * the first emitted token distributed as p_0 (the target alone);
  * P(N = k) = prod_{i<k} alpha_i * (1 - alpha_k) for k < gamma, prod_i alpha_i for k = gamma,
    with alpha_i = sum_x min(p_i(x), q_i(x)) (Eq. (1)'s acceptance rate per position);
  * after a rejection at k the emitted token distributed as norm(max(0, p_k - q_k)), and after
    full acceptance the bonus token distributed as p_gamma.
Each law is checked by a chi-square test at p > 1e-4; impossible tokens must never appear.
The draft-token sampler is checked the same way against softmax(logits / t)."""

import numpy as np
import pytest
import torch
from scipy import stats

from kv_sparse_speculative_amd import kvss

pytestmark = pytest.mark.gpu

V, GAMMA, B, CALLS = 8, 3, 32768, 32


def _softmax(z):
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _chi2(counts, probs, what):
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.sum()
    live = probs > 0
    assert np.all(counts[~live] == 0), f"{what}: impossible outcomes drawn"
    exp = probs[live] / probs[live].sum() * n
    pv = stats.chisquare(counts[live], exp).pvalue
    print(f"{what}: n={int(n)} p-value {pv:.3g}")
    assert pv > 1e-4, what


def test_speculative_sampling_law_on_the_gpu():
    rng = np.random.default_rng(77)
    zt = rng.normal(0.0, 1.5, size=(GAMMA + 1, V)).astype(np.float32)
    # a draft close to the target (acceptance rates ~0.7), so every count N has many samples
    zd = (zt[:GAMMA] + rng.normal(0.0, 0.7, size=(GAMMA, V))).astype(np.float32)
    p = _softmax(zt.astype(np.float64))            # the law of the stored float32 logits
    q = _softmax(zd.astype(np.float64))
    alpha = np.minimum(p[:GAMMA], q).sum(axis=1)
    target = torch.from_numpy(np.broadcast_to(zt, (B, GAMMA + 1, V)).copy()).cuda()
    draft = torch.from_numpy(np.broadcast_to(zd, (B, GAMMA, V)).copy()).cuda()

    first = np.zeros(V, dtype=np.int64)
    n_hist = np.zeros(GAMMA + 1, dtype=np.int64)
    emitted = np.zeros((GAMMA + 1, V), dtype=np.int64)        # token at position N, given N
    for c in range(CALLS):
        toks = np.stack([rng.choice(V, size=B, p=q[i]) for i in range(GAMMA)], axis=1)
        t_toks = torch.from_numpy(toks.astype(np.int32)).cuda()
        out, n_acc, _ = kvss.spec_accept(target, draft, t_toks, 1.0, seed=2024, offset=c)
        torch.cuda.synchronize()
        out, n_acc = out.cpu().numpy(), n_acc.cpu().numpy()
        assert np.all(out[np.arange(B), n_acc] >= 0)
        np.testing.assert_array_equal(out[:, :GAMMA][np.arange(GAMMA)[None, :] < n_acc[:, None]],
                                      toks[np.arange(GAMMA)[None, :] < n_acc[:, None]])
        first += np.bincount(out[:, 0], minlength=V)
        n_hist += np.bincount(n_acc, minlength=GAMMA + 1)
        for k in range(GAMMA + 1):
            sel = n_acc == k
            emitted[k] += np.bincount(out[sel, k], minlength=V)

    _chi2(first, p[0], "first emitted token ~ p_0")
    pn = np.empty(GAMMA + 1)
    reach = 1.0
    for k in range(GAMMA):
        pn[k] = reach * (1.0 - alpha[k])
        reach *= alpha[k]
    pn[GAMMA] = reach
    _chi2(n_hist, pn, "accepted count ~ Eq. (1) law")
    for k in range(GAMMA):
        r = np.maximum(p[k] - q[k], 0.0)
        _chi2(emitted[k], r / r.sum(), f"token after a rejection at {k} ~ norm(max(0, p - q))")
    _chi2(emitted[GAMMA], p[GAMMA], "bonus token after full acceptance ~ p_gamma")


@pytest.mark.parametrize("temp", [1.0, 0.6])
def test_draft_sampler_law_on_the_gpu(temp):
    """draft_sample at temperature t draws from softmax(logits / t): 2^20 draws, chi-square."""
    rng = np.random.default_rng(78)
    z = rng.normal(0.0, 1.5, size=V).astype(np.float32)
    p = _softmax(z.astype(np.float64) / temp)
    logits = torch.from_numpy(np.broadcast_to(z, (B, V)).copy()).cuda()
    counts = np.zeros(V, dtype=np.int64)
    for c in range(CALLS):
        tok, _ = kvss.draft_sample(logits, temp, seed=99, offset=c, step=1)
        torch.cuda.synchronize()
        counts += np.bincount(tok.cpu().numpy(), minlength=V)
    _chi2(counts, p, f"draft token at t={temp} ~ softmax(z / t)")
