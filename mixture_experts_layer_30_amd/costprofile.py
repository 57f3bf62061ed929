"""Per-expert cost profile of the TEMPO page (section "Dwa reżimy, jeden próg").

The page describes an expert's decode time with two regimes: below a token
threshold n* the time is set by streaming the expert's weights from HBM, once
per activated replica, whatever the number of tokens; above it by the grouped
GEMM's arithmetic, linear in the tokens (with the M dimension rounded to the
128-row tile).  One max-affine profile covers both:

    t(G, N) = max(a + b*G, c + beta*N)

with G the activated replicas and N the tokens.  On one GPU the replicas are
G distinct copies of one expert's weights sharing the N tokens evenly; the
threshold for G replicas is where the two pieces meet,
n*(G) = (a + b*G - c) / beta.  The page reports n* of about 156-168 tokens.

Fitting a max of two affine functions by least squares is not a linear
problem.  The reading taken here is the usual alternating scheme for
max-affine regression: assign each point to the piece that is larger there,
refit each piece by linear least squares on its points, repeat until the
assignment is stable; started from every split of the points by a threshold
on N, keeping the fit with the smallest squared error.  This module is plain
host arithmetic on measured times: no kernels.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class MaxAffineFit:
    a: float
    b: float
    c: float
    beta: float
    sse: float
    r2: float
    max_rel_err: float
    n_memory: int   # points where the memory piece is the larger one
    n_compute: int

    def predict(self, G, N):
        G = np.asarray(G, dtype=np.float64)
        N = np.asarray(N, dtype=np.float64)
        return np.maximum(self.a + self.b * G, self.c + self.beta * N)

    def n_star(self, G=1) -> Optional[float]:
        """Tokens at which the compute piece overtakes the memory piece for G
        replicas (None when the fit has no compute piece)."""
        if not self.beta > 0:
            return None
        return (self.a + self.b * G - self.c) / self.beta


def _lstsq(x, y):
    """(intercept, slope) of y ~ p + q x; slope 0 when x does not vary."""
    if len(y) == 0:
        return 0.0, 0.0
    if np.ptp(x) == 0:
        return float(np.mean(y)), 0.0
    A = np.stack([np.ones_like(x), x], axis=1)
    (p, q), *_ = np.linalg.lstsq(A, y, rcond=None)
    return float(p), float(q)


def _refine(G, N, t, mem):
    """Alternating refits from an initial assignment (True = memory piece)."""
    a = b = c = beta = 0.0
    for _ in range(100):
        a, b = _lstsq(G[mem], t[mem]) if mem.any() else (-np.inf, 0.0)
        c, beta = _lstsq(N[~mem], t[~mem]) if (~mem).any() else (-np.inf, 0.0)
        new = (a + b * G) >= (c + beta * N)
        if np.array_equal(new, mem):
            break
        mem = new
    pred = np.maximum(a + b * G, c + beta * N)
    return a, b, c, beta, float(np.sum((pred - t) ** 2)), mem


def fit_max_affine(G, N, t) -> MaxAffineFit:
    """Least-squares fit of t = max(a + b*G, c + beta*N) to measured points."""
    G = np.asarray(G, dtype=np.float64).ravel()
    N = np.asarray(N, dtype=np.float64).ravel()
    t = np.asarray(t, dtype=np.float64).ravel()
    if not (len(G) == len(N) == len(t)) or len(t) < 2:
        raise ValueError("need at least two (G, N, t) points of equal length")
    best = None
    for thr in np.unique(N):
        fit = _refine(G, N, t, N <= thr)
        if best is None or fit[4] < best[4] - 1e-12 * max(1.0, best[4]):
            best = fit
    a, b, c, beta, sse, mem = best
    if not mem.any():          # one affine piece in N only
        a, b = -np.inf, 0.0
    if mem.all():              # one affine piece in G only
        c, beta = -np.inf, 0.0
    pred = np.maximum(a + b * G, c + beta * N)
    ss_tot = float(np.sum((t - t.mean()) ** 2))
    r2 = 1.0 - sse / ss_tot if ss_tot > 0 else 1.0
    rel = float(np.max(np.abs(pred - t) / np.abs(t))) if np.all(t != 0) else float("nan")
    return MaxAffineFit(a, b, c, beta, sse, r2, rel, int(mem.sum()), int((~mem).sum()))
