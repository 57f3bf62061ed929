"""Pins of the analytic tax model (host arithmetic; no GPU).

The model follows the talk notes' BBB section (E_active under uniform routing)
and Section 5.3 (roofline latency with a padding factor eta).  Each pin is a
closed form of the definitions, a limit, or a Monte-Carlo estimate from the
oracle's own routing, so a dropped term, a swapped operand or a wrong exponent
fails one of them.
"""
import math

import numpy as np
import pytest

import oracle
from mixture_experts_layer_30_amd import configs, synth, taxmodel as tm
from mixture_experts_layer_30_amd.configs import LayerShape

MIX = configs.CONFIGS["mixtral"]
DS = configs.CONFIGS["deepseek_v3"]


def test_e_active_closed_forms():
    assert tm.e_active_uniform(0, 2, 8) == 0.0
    assert tm.e_active_uniform(1, 2, 8) == pytest.approx(2.0)           # one token: exactly K experts
    assert tm.e_active_uniform(1, 8, 256) == pytest.approx(8.0)
    assert tm.e_active_uniform(3, 8, 8) == pytest.approx(8.0)           # K = E: every expert
    assert tm.e_active_uniform(10 ** 6, 2, 8) == pytest.approx(8.0)     # saturates at E
    # two tokens, K of E: E(1 - (1-K/E)^2) = 2K - K^2/E
    assert tm.e_active_uniform(2, 2, 8) == pytest.approx(4 - 4 / 8)


def test_e_active_matches_oracle_routing_monte_carlo():
    """Uniform N(0,1) logits through the oracle's router: mean active experts
    within 4 standard errors of the closed form."""
    T, E, K, n = 16, 32, 4, 200
    counts = []
    for s in range(n):
        ids, _ = oracle.route(synth.router_logits(T, E, "uniform", seed=1000 + s), K)
        counts.append(len(np.unique(ids)))
    counts = np.asarray(counts, dtype=np.float64)
    se = counts.std(ddof=1) / math.sqrt(n)
    assert abs(counts.mean() - tm.e_active_uniform(T, K, E)) <= 4 * se


def test_single_token_has_no_tax_when_memory_bound():
    """m = 1, no shared experts: the MoE layer reads exactly the K experts' weights
    DenseFA holds, so both are bandwidth-bound on the same bytes: tau = 1."""
    r = tm.tax(MIX, 1)
    assert r["regime"] == "memory"
    assert r["tau_fa"] == pytest.approx(1.0, rel=1e-12)


def test_memory_bound_tau_is_bytes_ratio():
    m = 8
    ea = tm.e_active_uniform(m, MIX.topk, MIX.experts)
    r = tm.tax(MIX, m)
    H, I, K = MIX.hidden, MIX.inter, MIX.topk
    want = (ea * 3 * H * I * 2 + 2 * m * H * 2) / (3 * H * K * I * 2 + 2 * m * H * 2)
    assert r["regime"] == "memory"
    assert r["tau_fa"] == pytest.approx(want, rel=1e-12)
    # weight amplification: bounded by E/K, reached as every expert activates
    assert r["tau_fa"] < MIX.experts / MIX.topk


def test_compute_bound_tau_is_eta():
    """Huge batches: both layers compute-bound on equal flops, tau = eta."""
    r = tm.tax(MIX, 10 ** 7)
    assert r["regime"] == "compute"
    assert r["eta"] == tm.ETA_PREFILL
    assert r["tau_fa"] == pytest.approx(tm.ETA_PREFILL, rel=1e-9)
    r1 = tm.tax(MIX, 10 ** 7, eta=1.0)
    assert r1["tau_fa"] == pytest.approx(1.0, rel=1e-9)


def test_decode_bell_then_prefill_decline():
    """tau rises from 1 at one token towards E/K while both layers are bandwidth-
    bound, then falls towards eta once they are compute-bound (one eta for the
    whole sweep: the default switches from the decode to the prefill constant
    with the MoE layer's regime, a step of its own)."""
    ms = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 16384, 65536]
    taus = [tm.tax(MIX, m, eta=tm.ETA_PREFILL)["tau_fa"] for m in ms]
    peak = int(np.argmax(taus))
    assert 0 < peak < len(ms) - 1
    assert all(a <= b + 1e-12 for a, b in zip(taus[:peak], taus[1:peak + 1]))
    assert all(a >= b - 1e-12 for a, b in zip(taus[peak:], taus[peak + 1:]))
    assert taus[0] == pytest.approx(1.0)
    assert taus[-1] == pytest.approx(tm.ETA_PREFILL, rel=1e-6)
    regimes = [tm.tax(MIX, m)["regime"] for m in ms]
    assert regimes[0] == "memory" and regimes[-1] == "compute"
    assert "transition" in regimes


def test_densepa_is_the_all_experts_bound():
    """DensePA holds every expert: once all experts are active and the layer is
    bandwidth-bound, MoE and DensePA read the same weights (tau_pa -> 1)."""
    r = tm.tax(MIX, 64, e_active=MIX.experts)
    assert r["regime"] in ("memory", "transition")
    assert r["tau_pa"] == pytest.approx(1.0, rel=1e-9)
    # and with fewer experts active the MoE layer is cheaper than DensePA
    assert tm.tax(MIX, 4)["tau_pa"] < 1.0


def test_shared_experts_enter_both_sides():
    """A shared expert adds the same weights and flops to the MoE layer and to
    DenseFA (I_fa = K*I + I_s): at one token the tax stays 1."""
    sh = LayerShape("s", 1024, 512, 16, 2, 768, "bf16", (1,), ("uniform",))
    assert tm.tax(sh, 1)["tau_fa"] == pytest.approx(1.0, rel=1e-12)
    assert tm.dense_cost(sh, 5, sh.dense_fa_inter).flops == pytest.approx(
        tm.moe_cost(sh, 5, 3).flops)


def test_fine_grained_experts_amplify_more():
    """At the same batch DeepSeek-shaped experts (E=256, K=8) are amplified more
    than Mixtral-shaped ones (E=8, K=2): E_active/K can reach 32 instead of 4."""
    assert tm.tax(DS, 128)["tau_fa"] > tm.tax(MIX, 128)["tau_fa"]
