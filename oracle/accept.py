"""Speculative acceptance: greedy and rejection sampling (oracle, test infrastructure).

MagicDec Section 3.1 takes the speculative-decoding procedure of Leviathan et al.: the draft
proposes gamma tokens, the target scores gamma + 1 positions in one pass, and Eq. (1) gives
the expected number of emitted tokens, Omega(gamma, alpha) = (1 - alpha^(gamma+1)) /
(1 - alpha), for a per-position acceptance rate alpha. Section 5.1 (Setup) runs every
end-to-end experiment with greedy decoding. The paper does not print the acceptance rule;
the readings taken here:

Greedy (temperature 0). Draft token x_i is accepted while it equals the target's argmax at
position i (ties go to the lowest token id). At the first mismatch i the target's argmax at
i is emitted instead; if all gamma drafts match, the target's argmax at position gamma is
appended. So 1 .. gamma + 1 tokens are emitted.

Rejection sampling (temperature t > 0). p_i = softmax(target_i / t), q_i = softmax(draft_i / t).
Position i < gamma accepts x_i when u_i < p_i(x_i) / q_i(x_i), u_i a uniform in (0, 1). At the
first rejection i the emitted token is drawn from the residual max(0, p_i - q_i) (or from p_i
when the residual is all zero); if every draft token is accepted, an extra token is drawn
from p_gamma. Draws use an exponential race: token y = argmin_x E_x / w(x) over w(x) > 0 with
E_x = -log u'_x, which selects y with probability w(y) / sum w (ties: lowest id). The
uniforms come from the Philox layout of oracle.philox.

Outputs: out_tokens int32 [B, gamma + 1] (emitted tokens, then -1), num_accepted int32 [B]
(the number of accepted draft tokens, 0 .. gamma).
"""

import numpy as np

from .philox import accept_uniform, draft_uniforms, race_uniforms


def softmax(z, temperature):
    """softmax(z / temperature) in float64."""
    x = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def argmax_lowest(z):
    """Index of the maximum over the non-NaN entries, the lowest index on ties; -1 when the row
    holds no such entry (a reading: the pages take argmax over well-formed logits only)."""
    z = np.asarray(z)
    ok = ~np.isnan(z)
    if not ok.any():
        return -1
    return int(np.flatnonzero(ok & (z == z[ok].max()))[0])


def exponential_race(weights, u):
    """argmin_x (-log u_x) / weights_x over weights_x > 0; ties to the lowest x."""
    weights = np.asarray(weights, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    live = weights > 0
    keys = np.full(weights.shape, np.inf)
    with np.errstate(over="ignore"):      # a subnormal weight gives key +inf: it cannot win
        keys[live] = -np.log(u[live]) / weights[live]
    return argmax_lowest(-keys)


def greedy_accept(target, tokens):
    """Greedy acceptance. target [B, gamma + 1, V]; tokens [B, gamma]."""
    B, T, _ = target.shape
    gamma = T - 1
    out = np.full((B, T), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    for b in range(B):
        i = 0
        while i < gamma and argmax_lowest(target[b, i]) == int(tokens[b, i]):
            out[b, i] = tokens[b, i]
            i += 1
        out[b, i] = argmax_lowest(target[b, i])
        n_acc[b] = i
    return out, n_acc


def rejection_accept_one(p_rows, q_rows, tokens, u_accept, race_u):
    """Rejection sampling for one sequence from its probability rows.

    p_rows [gamma + 1, V] and q_rows [gamma, V] are target and draft probabilities;
    u_accept(i) gives the acceptance uniform of position i and race_u(i) the race uniforms
    [V] at emitting position i. Returns (emitted token list, number accepted).
    """
    gamma = q_rows.shape[0]
    emitted = []
    for i in range(gamma):
        x = int(tokens[i])
        if u_accept(i) < p_rows[i, x] / q_rows[i, x]:
            emitted.append(x)
            continue
        residual = np.maximum(p_rows[i] - q_rows[i], 0.0)
        if residual.sum() == 0.0:
            residual = p_rows[i]
        emitted.append(exponential_race(residual, race_u(i)))
        return emitted, i
    emitted.append(exponential_race(p_rows[gamma], race_u(gamma)))
    return emitted, gamma


def rejection_accept(target, draft, tokens, temperature, seed, offset, seq_ids=None):
    """Rejection-sampling acceptance with Philox uniforms.

    target [B, gamma + 1, V], draft [B, gamma, V] logits; tokens [B, gamma]. seq_ids gives the
    batch index each row had in the full batch (it enters the Philox counter); default 0..B-1.
    """
    B, T, V = target.shape
    gamma = T - 1
    ids = list(range(B)) if seq_ids is None else [int(x) for x in seq_ids]
    out = np.full((B, T), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    for b in range(B):
        p_rows = np.stack([softmax(target[b, i], temperature) for i in range(T)])
        q_rows = (np.stack([softmax(draft[b, i], temperature) for i in range(gamma)])
                  if gamma > 0 else np.zeros((0, V)))        # gamma = 0: only the draw from p_0
        sid = ids[b]
        emitted, n = rejection_accept_one(
            p_rows, q_rows, tokens[b],
            lambda i, sid=sid: accept_uniform(seed, offset, sid, i),
            lambda i, sid=sid: race_uniforms(seed, offset, sid, i, V))
        out[b, : len(emitted)] = emitted
        n_acc[b] = n
    return out, n_acc


def spec_accept(target, draft, tokens, temperature, seed=0, offset=0, seq_ids=None):
    """Greedy when temperature == 0, rejection sampling otherwise."""
    if temperature == 0:
        return greedy_accept(target, tokens)
    return rejection_accept(target, draft, tokens, temperature, seed, offset, seq_ids)


def draft_sample(logits, temperature, seed=0, offset=0, step=0, seq_ids=None):
    """The draft token of one draft step from the draft's logits [B, V].

    MagicDec Section 3.1: the draft proposes gamma tokens that the target then verifies with
    the rule above; Section 5.1 drafts greedily. Reading: temperature 0 takes the argmax (ties
    to the lowest id); temperature t > 0 draws from q = softmax(logits / t) by the same
    exponential race as the emitted token, with the uniforms of oracle.philox.draft_uniforms
    (a stream of its own, at position `step`). Returns int32 [B].
    """
    logits = np.asarray(logits)
    B, V = logits.shape
    ids = list(range(B)) if seq_ids is None else [int(x) for x in seq_ids]
    out = np.empty(B, dtype=np.int32)
    for b in range(B):
        if temperature == 0:
            out[b] = argmax_lowest(logits[b])
        else:
            out[b] = exponential_race(softmax(logits[b], temperature),
                                      draft_uniforms(seed, offset, ids[b], step, V))
    return out

