"""CPU checks of the speedup model against the paper's equations, its printed rows and the
model's own limits: Eq. (1) against the geometric series it sums and its inverse, Eq. (2) in
its degenerate cases and against every printed Table 2 / Table 4 row (tests/golden), the layer
size against Llama-3.1-8B's published parameter count, and the Section 3.2 regime behaviour."""

import math
import os

import pytest

from kv_sparse_speculative_amd.speedup_model import (LLAMA8B_LAYER, LayerModel, alpha_from_omega,
                                                     best_gamma, curves, layer_params, omega,
                                                     s_inflection, sd_cost_ratio,
                                                     sd_time_per_token)

RATES = {"attn_decode_Bps": 5.7e12, "attn_verify_Bps": 5.8e12, "attn_draft_Bps": 5.7e12,
         "draft_fixed_s": 12e-6, "stream_Bps": 6.15e12, "select_dynamic_Bps": 2.9e12}

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "magicdec_speedup_rows.txt")


def _printed_rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        t, pre, bsz, g, gtd, tv, om, tar, tsd, x = line.split()
        rows.append((t, int(pre), int(bsz), int(g), float(gtd), float(tv), float(om), float(tar),
                     float(tsd), float(x)))
    return rows


def test_printed_rows_follow_eq2():
    """Each printed row: T^SD is Eq. (2)'s (gamma T_D + T_V) / Omega plus the non-model overhead
    (0.7-3.5% on these rows), and the printed speedup is T^AR / T^SD to two decimals."""
    rows = _printed_rows()
    assert len(rows) == 9
    for t, pre, bsz, g, gtd, tv, om, tar, tsd, x in rows:
        pred = sd_time_per_token(gtd, tv, om)
        assert 0.0 <= (tsd - pred) / pred <= 0.04, (t, pre, bsz, pred, tsd)
        assert round(tar / tsd, 2) == x, (t, pre, bsz, tar / tsd, x)
        # the same through Eq. (2) in the model's form: T^SD / T^AR, alpha from Omega (Eq. (1))
        a = alpha_from_omega(g, om)
        assert 0.0 < a < 1.0 and omega(g, a) == pytest.approx(om, rel=1e-12)
        ratio = sd_cost_ratio(g, a, gtd / g, tv, tar)
        assert ratio == pytest.approx(pred / tar, rel=1e-9)
        assert 1.0 / ratio == pytest.approx(x, rel=0.045)


def test_printed_table4_speedup_grows_with_batch():
    """Table 4 (32000-token prefill, batches 16 / 32 / 64): the speedup grows with batch size,
    the Section 3.2 regime above the critical length."""
    t4 = [r for r in _printed_rows() if r[0] == "table4"]
    assert [r[2] for r in t4] == [16, 32, 64]
    assert t4[0][9] < t4[1][9] < t4[2][9]


def test_alpha_from_omega_inverts_eq1():
    for g in (1, 3, 7, 11):
        for a in (0.0, 0.25, 0.7, 0.95):
            assert alpha_from_omega(g, omega(g, a)) == pytest.approx(a, abs=1e-9)
    with pytest.raises(ValueError):
        alpha_from_omega(3, 4.5)


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


def test_curves_cover_the_batches_and_grow_with_context():
    m = LayerModel(LLAMA8B_LAYER, RATES)
    c = curves(m, 512, (0.8,))
    assert set(c["0.8"]) == {"16", "32", "64", "128", "256"}
    for B, pts in c["0.8"].items():
        sp = [p[2] for p in pts]
        assert all(x < y for x, y in zip(sp, sp[1:])), B     # longer contexts gain more
    # above the inflection the largest batch gains most
    s_inf = s_inflection(m, 512, 0.8)
    long = [p for p in c["0.8"]["256"] if p[0] >= 2 * s_inf][0][2]
    small = [p for p in c["0.8"]["16"] if p[0] >= 2 * s_inf][0][2]
    assert long > small
