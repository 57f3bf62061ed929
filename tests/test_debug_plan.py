"""The MOE_DEBUG plan checker (host logic, no GPU): alignments the oracle builds
pass it, and each planted mistake in one of the five arrays is named."""
import numpy as np
import pytest

import oracle
from mixture_experts_layer_30_amd import synth
from mixture_experts_layer_30_amd.debug import PlanError, check_plan, debug_enabled


def cases():
    # (ids [T][K], E, B, pad): even routing, skewed routing with empty experts,
    # a single token, max padding, unused slots of a per-token budget
    rng = np.random.default_rng(5)
    z = oracle.route(synth.router_logits(40, 16, "zipf"), 4)[0]
    u = oracle.route(synth.router_logits(64, 8, "uniform"), 2)[0]
    one = oracle.route(synth.router_logits(1, 64, "zipf"), 8)[0]
    var = z.copy()
    var[rng.random(var.shape) < 0.3] = -1
    return [(u, 8, 16, "block"), (z, 16, 64, "block"), (one, 64, 16, "block"),
            (z, 16, 16, "max"), (var, 16, 32, "block")]


def build(ids, E, B, pad):
    T, K = ids.shape
    if pad == "block":
        cap = (T * K + min(E, T * K) * (B - 1) + B - 1) // B * B
    else:
        cap = E * ((T + B - 1) // B) * B
    return oracle.align(ids, E, B, cap, mode=pad), cap


@pytest.mark.parametrize("case", range(5))
def test_oracle_plans_pass(case):
    ids, E, B, pad = cases()[case]
    plan, cap = build(ids, E, B, pad)
    check_plan(plan, ids, E, B, cap, pad)


def _mutations(plan, ids):
    """(name, array, mutate) for one planted mistake per array and invariant."""
    T, K = ids.shape
    def swap_rows(a):
        e = int(np.argmax(plan["expert_counts"]))
        r = int(plan["expert_offsets"][e])
        a[r], a[r + 1] = a[r + 1], a[r]
    def drop_pair(a):
        e = int(np.argmax(plan["expert_counts"]))
        a[int(plan["expert_offsets"][e])] = T * K
    def pad_row(a):
        a[-1] = 0          # a padding row past the total that names a pair
    return [
        ("count", "expert_counts", lambda a: a.__setitem__(int(np.argmax(a)), a.max() - 1)),
        ("offset", "expert_offsets", lambda a: a.__setitem__(1, a[1] + 1)),
        ("order", "sorted_ids", swap_rows),
        ("lost pair", "sorted_ids", drop_pair),
        ("sentinel", "sorted_ids", pad_row),
        ("block", "block_expert", lambda a: a.__setitem__(0, (a[0] + 1) % 3)),
        ("tail block", "block_expert", lambda a: a.__setitem__(-1, 0)),
        ("inverse", "inv_pos", lambda a: a.__setitem__(int(np.argmax(a >= 0)), a[np.argmax(a >= 0)] + 1)),
    ]


@pytest.mark.parametrize("case", [0, 1, 4])
def test_planted_mistakes_are_named(case):
    ids, E, B, pad = cases()[case]
    plan, cap = build(ids, E, B, pad)
    for name, key, mutate in _mutations(plan, ids):
        bad = {k: v.copy() for k, v in plan.items()}
        mutate(bad[key])
        if np.array_equal(bad[key], plan[key]):
            continue   # (no-op on this plan, e.g. no padding row to corrupt)
        with pytest.raises(PlanError):
            check_plan(bad, ids, E, B, cap, pad)


def test_shapes_and_routing_checked():
    ids, E, B, pad = cases()[0]
    plan, cap = build(ids, E, B, pad)
    with pytest.raises(PlanError):
        check_plan({**plan, "inv_pos": plan["inv_pos"][:-1]}, ids, E, B, cap, pad)
    other = ids.copy()
    other[0, 0] = (other[0, 0] + 1) % E if (other[0, 0] + 1) % E not in other[0] else other[0, 0]
    other[0, 1] = (other[0, 1] + 3) % E
    with pytest.raises(PlanError):   # the plan of different routing
        check_plan(plan, other, E, B, cap, pad)


def test_debug_flag(monkeypatch):
    monkeypatch.delenv("MOE_DEBUG", raising=False)
    assert not debug_enabled()
    monkeypatch.setenv("MOE_DEBUG", "1")
    assert debug_enabled()
    assert not debug_enabled(False)
    monkeypatch.setenv("MOE_DEBUG", "0")
    assert not debug_enabled() and debug_enabled(True)
