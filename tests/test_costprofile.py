"""Max-affine per-expert cost profile (TEMPO page, section "Dwa reżimy, jeden
próg"): the fit recovers known profiles and the threshold n* is where the
two pieces meet."""
import numpy as np
import pytest

from mixture_experts_layer_30_amd.costprofile import fit_max_affine

GS = [1, 2, 4, 8]
NS = [1, 2, 4, 8, 16, 32, 64, 96, 128, 160, 192, 256, 384, 512, 768, 1024]


def grid(a, b, c, beta, noise=0.0, seed=0):
    rng = np.random.default_rng(seed)
    G, N, t = [], [], []
    for g in GS:
        for n in NS:
            if n < g:
                continue
            v = max(a + b * g, c + beta * n)
            G.append(g)
            N.append(n)
            t.append(v * (1.0 + noise * rng.standard_normal()))
    return np.array(G), np.array(N), np.array(t)


def test_exact_profile_recovered():
    # memory piece 30 us + 40 us per replica, compute 5 us + 0.5 us per token
    G, N, t = grid(30.0, 40.0, 5.0, 0.5)
    f = fit_max_affine(G, N, t)
    assert f.a == pytest.approx(30.0, abs=1e-6)
    assert f.b == pytest.approx(40.0, abs=1e-6)
    assert f.c == pytest.approx(5.0, abs=1e-6)
    assert f.beta == pytest.approx(0.5, abs=1e-9)
    assert f.sse < 1e-12 and f.r2 == pytest.approx(1.0)
    # the threshold is where the pieces meet: (a + b G - c) / beta
    assert f.n_star(1) == pytest.approx((30 + 40 - 5) / 0.5)
    assert f.n_star(8) == pytest.approx((30 + 320 - 5) / 0.5)
    n1 = f.n_star(1)
    assert f.predict(1, n1 - 1) == pytest.approx(70.0)
    assert f.predict(1, n1 + 10) == pytest.approx(5 + 0.5 * (n1 + 10))


def test_noisy_profile_close():
    G, N, t = grid(30.0, 40.0, 5.0, 0.5, noise=0.01, seed=3)
    f = fit_max_affine(G, N, t)
    assert f.b == pytest.approx(40.0, rel=0.05)
    assert f.beta == pytest.approx(0.5, rel=0.05)
    assert f.n_star(1) == pytest.approx(130.0, rel=0.08)
    assert f.r2 > 0.99 and f.max_rel_err < 0.05


def test_piece_assignment_follows_the_max():
    G, N, t = grid(30.0, 40.0, 5.0, 0.5)
    f = fit_max_affine(G, N, t)
    mem = (30 + 40 * G) >= (5 + 0.5 * N)
    assert f.n_memory == int(mem.sum()) and f.n_compute == int((~mem).sum())


def test_memory_only_has_no_threshold():
    G = np.array([1, 2, 4, 8, 1, 2, 4, 8], dtype=float)
    N = np.array([8, 8, 8, 8, 16, 16, 16, 16], dtype=float)
    t = 10.0 + 20.0 * G
    f = fit_max_affine(G, N, t)
    assert f.n_star(1) is None
    assert f.b == pytest.approx(20.0) and f.a == pytest.approx(10.0)


def test_compute_only_is_linear_in_tokens():
    N = np.array([128, 256, 512, 1024, 2048], dtype=float)
    G = np.ones_like(N)
    t = 3.0 + 0.25 * N
    f = fit_max_affine(G, N, t)
    assert f.beta == pytest.approx(0.25) and f.c == pytest.approx(3.0)
    assert f.predict(1, 4096) == pytest.approx(3.0 + 0.25 * 4096)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        fit_max_affine([1], [1], [1.0])
    with pytest.raises(ValueError):
        fit_max_affine([1, 2], [1, 2, 3], [1.0, 2.0])
