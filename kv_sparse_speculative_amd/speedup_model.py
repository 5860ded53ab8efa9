"""Speculative-decoding speedup model for one MI355X, fed with the library's measured times.

MagicDec Section 3.1 gives the speedup of speculative decoding through
  Eq. (1)  Omega(gamma, alpha) = (1 - alpha^(gamma+1)) / (1 - alpha), the expected tokens per
           verification for per-token acceptance rate alpha,
  Eq. (2)  T_avg^SD / T_T = (gamma * T_D / T_T + T_V(gamma) / T_T) / Omega(gamma, alpha),
and Section 4.1 adds the selection cost of a sparse-KV draft,
  Eq. (3)  T_D,select = T_D(B, K) + T_select(B, S, K),
  Eq. (4)  minimise Eq. (2) with Eq. (3) over the strategy, K, gamma (alpha is the strategy's).
Section 3.2 explains the regime change this model reproduces: at long S the per-step cost is
the KV load, shared by verification and decoding (T_V / T_T -> 1), while a fixed-budget draft's
cost stays flat, so the speedup grows with batch size above a critical length S_inflection.

Per-layer times are a roofline of two terms for n query tokens per sequence and R cached rows:
  linear layers  max(weight bytes / read bandwidth, 2 * params * B * n / matrix-core rate)
  attention      B * R * (KV bytes per row) / attention bandwidth  (+ the measured fixed part)
The attention bandwidths come from bench.py's measurements on the GPU, one per call:
  T_T  a one-token decode over the whole cache (verify_attn_full with T = 1),
  T_V  the gamma + 1 token verify over the whole cache,
  T_D  the draft: its measured time at the measured (B, K), of which the part proportional to
       B * K runs at the decode rate and the rest is a fixed launch cost,
  T_select (dynamic Top-K) the search over the prefix, timed as the dynamic step minus the
       static draft.
The weight read uses the measured stream-read rate; the linear-layer compute uses the dense bf16
matrix-core peak (an optimistic bound, which favours the target at large batch). alpha cannot
be measured without trained weights and data, so it is swept.
"""

import math

# Llama-3.1-8B decoder layer: hidden 4096, MLP 14336, 32 query / 8 KV heads of 128 dims.
LLAMA8B_LAYER = {
    "hidden": 4096, "mlp": 14336, "q_heads": 32, "kv_heads": 8, "head_dim": 128, "layers": 32,
}
MFMA_BF16_PEAK = 2.5e15          # dense bf16 FLOP/s of one MI355X


def layer_params(arch):
    """Weights of one decoder layer (attention projections + gated MLP; norms are negligible)."""
    h, f = arch["hidden"], arch["mlp"]
    kv = arch["kv_heads"] * arch["head_dim"]
    q = arch["q_heads"] * arch["head_dim"]
    return h * q + 2 * h * kv + q * h + 3 * h * f


def omega(gamma, alpha):
    """Eq. (1): expected tokens per verification (gamma + 1 when every draft is accepted)."""
    if alpha >= 1.0:
        return gamma + 1.0
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def alpha_from_omega(gamma, om, tol=1e-13):
    """alpha with omega(gamma, alpha) = om (Eq. (1) increases with alpha), om in [1, gamma + 1]."""
    if not 1.0 <= om <= gamma + 1.0:
        raise ValueError(f"Omega {om} outside [1, {gamma + 1}]")
    lo, hi = 0.0, 1.0
    while hi - lo > tol:
        mid = 0.5 * (lo + hi)
        if omega(gamma, mid) < om:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def sd_time_per_token(gamma_t_draft, t_verify, om):
    """T_avg^SD = (gamma * T_D + T_V) / Omega (Section 3.1, the text before Eq. (2))."""
    return (gamma_t_draft + t_verify) / om


def sd_cost_ratio(gamma, alpha, t_draft, t_verify, t_target):
    """Eq. (2): T_avg^SD / T_T (speedup is its reciprocal)."""
    return sd_time_per_token(gamma * t_draft, t_verify, omega(gamma, alpha)) / t_target


class LayerModel:
    """Per-layer step times at batch B and context S from the measured rates.

    rates: attn_decode_Bps (one-token decode over the whole cache), attn_verify_Bps (gamma + 1
    token verify), attn_draft_Bps (the draft's per-row rate), draft_fixed_s (the measured draft
    launch's time not explained by its bytes at that rate), stream_Bps (plain read rate, used
    for weights), select_dynamic_Bps (the dynamic Top-K search's bandwidth over the prefix).
    """

    def __init__(self, arch, rates, bytes_per_elem=2):
        self.arch = arch
        self.rates = rates
        self.params = layer_params(arch)
        self.w_bytes = self.params * bytes_per_elem
        self.row = arch["kv_heads"] * arch["head_dim"] * 2 * bytes_per_elem   # K + V, one row

    def linear(self, B, n):
        return max(self.w_bytes / self.rates["stream_Bps"],
                   2.0 * self.params * B * n / MFMA_BF16_PEAK)

    def target(self, B, S):
        """T_T: one decode token per sequence over S + 1 rows."""
        return self.linear(B, 1) + B * (S + 1) * self.row / self.rates["attn_decode_Bps"]

    def verify(self, B, S, gamma):
        """T_V(gamma): gamma + 1 tokens per sequence over S + gamma + 1 rows (one KV read)."""
        return (self.linear(B, gamma + 1)
                + B * (S + gamma + 1) * self.row / self.rates["attn_verify_Bps"])

    def draft(self, B, K):
        """T_D(B, K): self-speculation (same weights) over a K-row sparse KV."""
        return (self.linear(B, 1) + self.rates["draft_fixed_s"]
                + B * K * self.row / self.rates["attn_draft_Bps"])

    def select_dynamic(self, B, S):
        """T_select of a per-step dynamic Top-K search: it reads K of the whole prefix."""
        return B * S * (self.row / 2) / self.rates["select_dynamic_Bps"]


def best_gamma(model, B, S, K, alpha, dynamic=False, gammas=range(1, 9)):
    """Eq. (4) for one strategy and alpha: (gamma_opt, speedup at gamma_opt)."""
    t_t = model.target(B, S)
    t_d = model.draft(B, K) + (model.select_dynamic(B, S) if dynamic else 0.0)
    best = None
    for g in gammas:
        x = 1.0 / sd_cost_ratio(g, alpha, t_d, model.verify(B, S, g), t_t)
        if best is None or x > best[1]:
            best = (g, x)
    return best


def s_inflection(model, K, alpha, batches=(16, 256), lengths=None):
    """Smallest context S at which the best speedup grows with batch size (Section 3.2)."""
    lengths = lengths or [2 ** e for e in range(8, 18)]
    for S in lengths:
        lo = best_gamma(model, batches[0], S, K, alpha)[1]
        hi = best_gamma(model, batches[1], S, K, alpha)[1]
        if hi > lo:
            return S
    return None


def rates_from_bench(calls, nxt, stream_gbs, wl_batch, wl_context, draft_rows):
    """Measured rates from bench.py's per-call results (bytes and ms) at one workload: the
    decode rate from the one-token decode over the whole cache, the verify rate from the verify
    call, the draft as its measured time split into a part proportional to its rows (at the
    decode rate) and a fixed remainder, the dynamic search from the dynamic Top-K step."""
    verify = calls["verify"]
    draft = calls["draft_snapkv"]
    attn_verify = verify["bytes"] / (verify["ms"] * 1e-3)
    dec = nxt.get("decode_full") if nxt else None
    attn_decode = dec["bytes"] / (dec["ms"] * 1e-3) if dec else attn_verify
    draft_s = draft["ms"] * 1e-3
    fixed = max(draft_s - draft["bytes"] / attn_decode, 0.0)
    rates = {
        "attn_decode_Bps": attn_decode,
        "attn_verify_Bps": attn_verify,
        "attn_draft_Bps": attn_decode,
        "draft_fixed_s": fixed,
        "stream_Bps": stream_gbs * 1e9,
        "draft_measured_Bps": draft["bytes"] / draft_s,
    }
    dyn = nxt.get("draft_topk_dynamic") if nxt else None
    if dyn:
        # the search time = dynamic step - static draft step; over the prefix K bytes
        search_s = max(dyn["ms"] - draft["ms"], 1e-9) * 1e-3
        prefix_k = wl_batch * wl_context * LLAMA8B_LAYER["kv_heads"] * LLAMA8B_LAYER["head_dim"] * 2
        rates["select_dynamic_Bps"] = prefix_k / search_s
    else:
        rates["select_dynamic_Bps"] = attn_verify / 2
    return rates


def curves(model, K, alphas, batches=(16, 32, 64, 128, 256),
           lengths=(1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072), dynamic=False):
    """Speedup against context length per batch size (Section 3.2, Figs. 2-3 style): for each
    alpha, {B: [[S, gamma_opt, speedup], ...]}."""
    out = {}
    for a in alphas:
        out[str(a)] = {str(B): [[S, *[round(v, 3) if isinstance(v, float) else v
                                      for v in best_gamma(model, B, S, K, a, dynamic=dynamic)]]
                                for S in lengths]
                       for B in batches}
    return out


def summary(rates, B, S, K_static=512, alphas=(0.6, 0.7, 0.8, 0.9, 0.95)):
    """The model at the measured point, per strategy and alpha; speedup-vs-S curves per batch
    size; S_inflection per alpha, and its sensitivity to taking T_T at the verify rate instead
    of the measured decode rate."""
    m = LayerModel(LLAMA8B_LAYER, rates)
    out = {
        "per_layer_us": {
            "T_T": round(m.target(B, S) * 1e6, 1),
            "T_V_gamma4": round(m.verify(B, S, 4) * 1e6, 1),
            "T_V_over_T_T": round(m.verify(B, S, 4) / m.target(B, S), 4),
            "T_D_static_K512": round(m.draft(B, K_static) * 1e6, 1),
            "T_select_dynamic": round(m.select_dynamic(B, S) * 1e6, 1),
            "weights_read": round(m.w_bytes / rates["stream_Bps"] * 1e6, 1),
        },
        "rates_GBps": {k[:-4]: round(v / 1e9, 1) for k, v in rates.items() if k.endswith("_Bps")},
        "draft_fixed_us": round(rates["draft_fixed_s"] * 1e6, 2),
        "speedup": {},
    }
    for name, dyn in (("static_K512", False), ("dynamic_topk_K512", True)):
        out["speedup"][name] = {
            str(a): [best_gamma(m, B, S, K_static, a, dynamic=dyn)[0],
                     round(best_gamma(m, B, S, K_static, a, dynamic=dyn)[1], 3)]
            for a in alphas
        }
    out["curves_static_K512"] = curves(m, K_static, (0.7, 0.8, 0.9))
    alt = LayerModel(LLAMA8B_LAYER, dict(rates, attn_decode_Bps=rates["attn_verify_Bps"]))
    out["S_inflection_K512"] = {
        str(a): {"measured_T_T": s_inflection(m, K_static, a),
                 "T_T_at_verify_rate": s_inflection(alt, K_static, a)}
        for a in (0.7, 0.8, 0.9)}
    return out
