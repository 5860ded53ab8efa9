"""CPU checks of the speedup model against the paper's equations and the model's own limits:
Eq. (1) against the geometric series it sums, Eq. (2) in its degenerate cases, the layer size
against Llama-3.1-8B's published parameter count, and the Section 3.2 regime behaviour."""

import math

import pytest

from kv_sparse_speculative_amd.speedup_model import (LLAMA8B_LAYER, LayerModel, best_gamma,
                                                     layer_params, omega, s_inflection,
                                                     sd_cost_ratio)

RATES = {"attn_verify_Bps": 5.8e12, "attn_draft_Bps": 5.8e12, "draft_fixed_s": 12e-6,
         "stream_Bps": 6.15e12, "select_dynamic_Bps": 2.9e12}


@pytest.mark.parametrize("gamma", [1, 3, 4, 8])
@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.8, 0.99, 1.0])
def test_omega_is_the_expected_accepted_run(gamma, alpha):
    assert omega(gamma, alpha) == pytest.approx(sum(alpha ** i for i in range(gamma + 1)))


def test_eq2_degenerate_cases():
    # free draft, verification as cheap as decoding: the speedup is Omega itself
    assert 1 / sd_cost_ratio(4, 0.8, 0.0, 1.0, 1.0) == pytest.approx(omega(4, 0.8))
    # nothing accepted: one verification per token, plus the wasted drafts
    assert sd_cost_ratio(3, 0.0, 0.1, 1.0, 1.0) == pytest.approx(1.3)


def test_layer_size_matches_llama_3_1_8b():
    a = LLAMA8B_LAYER
    vocab = 128256
    total = a["layers"] * layer_params(a) + 2 * vocab * a["hidden"]   # + embedding and LM head
    assert total == pytest.approx(8.03e9, rel=0.01)


def test_long_context_regime():
    """Section 3.2: as S grows the KV load dominates, T_V / T_T -> 1 and T_D / T_T -> 0."""
    m = LayerModel(LLAMA8B_LAYER, RATES)
    B = 64
    r_v = [m.verify(B, S, 4) / m.target(B, S) for S in (1000, 8000, 32000, 128000)]
    r_d = [m.draft(B, 512) / m.target(B, S) for S in (1000, 8000, 32000, 128000)]
    assert all(x >= y for x, y in zip(r_v, r_v[1:])) and r_v[-1] < 1.02
    assert all(x > y for x, y in zip(r_d, r_d[1:])) and r_d[-1] < 0.05
    # T_T is linear in S at fixed B (memory-bound attention)
    d1 = m.target(B, 20000) - m.target(B, 10000)
    d2 = m.target(B, 30000) - m.target(B, 20000)
    assert d1 == pytest.approx(d2)


def test_inflection_separates_the_two_regimes():
    m = LayerModel(LLAMA8B_LAYER, RATES)
    s_inf = s_inflection(m, 512, 0.8)
    assert s_inf is not None
    below, above = s_inf // 2, s_inf * 2
    assert best_gamma(m, 256, above, 512, 0.8)[1] > best_gamma(m, 16, above, 512, 0.8)[1]
    assert best_gamma(m, 256, below, 512, 0.8)[1] <= best_gamma(m, 16, below, 512, 0.8)[1]


def test_dynamic_selection_costs_more_than_static():
    m = LayerModel(LLAMA8B_LAYER, RATES)
    g_s, x_s = best_gamma(m, 64, 32000, 512, 0.9)
    g_d, x_d = best_gamma(m, 64, 32000, 512, 0.9, dynamic=True)
    assert x_d < x_s
