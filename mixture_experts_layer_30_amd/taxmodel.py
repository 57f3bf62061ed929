"""Analytic MoE-tax model (Balls-Bins-Buckets), evaluated with MI355X constants.

Follows the talk notes on "Demystifying the Mixture of Experts Serving Tax":

* section "BBB モデルの構成": m tokens each routed to K of E experts; under
  uniform routing the expected number of experts that receive at least one
  token is E * (1 - (1 - K/E)^m);
* section "分析モデルの検証 (Section 5.3)": a roofline-style latency per layer from
  the HBM bandwidth, the bf16 peak and a padding factor eta (constants for
  decode and prefill), which the pages report within 10-30 % of measurements
  and which separates a memory-bound, a compute-bound and a transition regime;
* section "定義": tau = T(MoE, b) / T(DenseFA, b), and DensePA as the dense FFN
  with the MoE's parameter count.

The reading taken where the notes leave the formula open: the layer time is
max(bytes / BW, eta * flops / P), with bytes = the weights of the experts that
are used (all of them for a dense FFN) plus the token rows in and out, and
flops = 2 per multiply-add of the SwiGLU; eta multiplies the compute term of
the MoE layer only (the dense FFN has no padding).  The three regimes of the
tax: "memory" when the MoE layer and DenseFA are both bandwidth-bound (tau is
then the ratio of bytes, about E_active / K), "compute" when both are
compute-bound (tau = eta), "transition" when they are bound differently.
This module is plain host arithmetic on shapes: no kernels.
"""
from dataclasses import dataclass

# MI355X public figures (HBM3E bandwidth, dense bf16 MFMA peak)
MI355X_HBM_BPS = 8.0e12
MI355X_BF16_FLOPS = 2.5e15
# padding factors of the notes' validation (section 5.3)
ETA_DECODE = 1.05
ETA_PREFILL = 1.25


def e_active_uniform(m, K, E):
    """Expected experts with >= 1 token when each of m tokens picks K of E uniformly."""
    if m <= 0:
        return 0.0
    return E * (1.0 - (1.0 - K / E) ** m)


@dataclass
class LayerCost:
    bytes: float
    flops: float


def moe_cost(shape, m, e_active, elem_bytes=2):
    """Bytes and flops of one MoE layer pass over m tokens with e_active experts used."""
    H, I, K, Is = shape.hidden, shape.inter, shape.topk, shape.shared_inter
    weights = (e_active * 3 * H * I + 3 * H * Is) * elem_bytes
    tokens_io = 2 * m * H * elem_bytes
    flops = 6.0 * m * K * H * I + 6.0 * m * H * Is
    return LayerCost(weights + tokens_io, flops)


def dense_cost(shape, m, inter, elem_bytes=2):
    """Bytes and flops of a dense SwiGLU FFN of width `inter` over m tokens."""
    H = shape.hidden
    return LayerCost(3.0 * H * inter * elem_bytes + 2 * m * H * elem_bytes, 6.0 * m * H * inter)


def layer_time(cost, bw, peak, eta=1.0):
    """(seconds, regime): max of the HBM and the (padded) compute term."""
    t_mem = cost.bytes / bw
    t_cmp = eta * cost.flops / peak
    return (t_mem, "memory") if t_mem >= t_cmp else (t_cmp, "compute")


def tax(shape, m, e_active=None, bw=MI355X_HBM_BPS, peak=MI355X_BF16_FLOPS, eta=None):
    """Predicted tau vs DenseFA and vs DensePA for m tokens.

    e_active defaults to the uniform-routing expectation; eta defaults to the
    notes' decode constant when the MoE layer is memory-bound and to the
    prefill constant when it is compute-bound.
    """
    ea = e_active_uniform(m, shape.topk, shape.experts) if e_active is None else e_active
    eb = 4 if shape.dtype == "f32" else 2
    moe = moe_cost(shape, m, ea, eb)
    if eta is None:
        _, reg = layer_time(moe, bw, peak, 1.0)
        eta = ETA_DECODE if reg == "memory" else ETA_PREFILL
    t_moe, reg_moe = layer_time(moe, bw, peak, eta)
    t_fa, reg_fa = layer_time(dense_cost(shape, m, shape.dense_fa_inter, eb), bw, peak)
    t_pa, reg_pa = layer_time(dense_cost(shape, m, shape.dense_pa_inter, eb), bw, peak)
    regime = reg_moe if reg_moe == reg_fa else "transition"
    return {"e_active": ea, "eta": eta, "t_moe_s": t_moe, "t_densefa_s": t_fa,
            "t_densepa_s": t_pa, "tau_fa": t_moe / t_fa, "tau_pa": t_moe / t_pa,
            "regime": regime, "moe_regime": reg_moe, "densefa_regime": reg_fa,
            "densepa_regime": reg_pa}
