"""Budgeted per-matrix bitrates and the reconstruction error they trade (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[ABS] selects each matrix's resolution from sampled storage estimates at an
arbitrary target rate; [README] 性能 and [NEWS] 官方基準 quote whole-model packs
at one average rate (2.3 / 3.0 bpp over the 276 layers of a diffusion
transformer).  The pages do not say how bits are spread over matrices; this
reading spends a total bit budget on one candidate target per matrix so that
the summed (caller-weighted) squared reconstruction error is small, using only
the weights themselves (data-free):

* ``distortion``: squared error of the lattice reconstruction fl32(h_r u)
  against the input and the input's squared norm.  Pinned (tests) against the
  FP32-container decode, whose output is exactly fl32(h_r u), and against the
  E8 second moment at high rate.
* ``plan``: per matrix the candidate minimising cost + lambda bits (ties: fewer
  bits, then the lower index); lambda = 0 if that fits the budget, else the
  smallest of the values (c_j - c_k) / (b_k - b_j) at which some matrix's pick
  changes whose pick fits (none may, when c + lambda b rounds a tie at the largest
  such value to the wider side: then the fewest bits everywhere, ties by lower
  cost and index, the large-lambda limit); then upgrades, one at a time, to the candidate with
  the most cost saved per extra bit that still fits (ties: lower matrix, lower
  candidate).  Pinned against brute force over every combination on small
  instances at the budgets the Lagrangian step lands on exactly (there it is
  optimal), and by feasibility.
"""
from __future__ import annotations

import numpy as np

from .codec import parse_blob, decode
from .numerics import source_to_f64
from .rate import half_steps


def distortion(src, dtype: int, blob: bytes):
    """(sum (w - fl32(h_r u))^2, sum w^2) over all entries, in float64."""
    b = parse_blob(blob)
    u, _, _ = decode(blob)
    w = source_to_f64(np.asarray(src), dtype).reshape(b.R, b.C)
    h = half_steps(b.s_bits, b.delta)
    wh = (h[:, None] * u.astype(np.float32)).astype(np.float32).astype(np.float64)
    d = w - wh
    return float(np.sum(d * d)), float(np.sum(w * w))


class Infeasible(ValueError):
    pass


def _pick(bits, cost, lam):
    n, m = bits.shape
    ch = []
    for i in range(n):
        best, bv = 0, cost[i, 0] + lam * bits[i, 0]
        for j in range(1, m):
            v = cost[i, j] + lam * bits[i, j]
            if v < bv or (v == bv and bits[i, j] < bits[i, best]):
                best, bv = j, v
        ch.append(best)
    return ch


def _used(bits, ch):
    t = 0.0
    for i, j in enumerate(ch):
        t += bits[i, j]
    return t


def plan(bits, cost, budget):
    """Candidate index per matrix (see the module docstring)."""
    bits = np.asarray(bits, dtype=np.float64)
    cost = np.asarray(cost, dtype=np.float64)
    n, m = bits.shape
    least = 0.0
    for i in range(n):
        least += float(bits[i].min())
    if least > budget:
        raise Infeasible("budget below the smallest candidates")
    ch = _pick(bits, cost, 0.0)
    if _used(bits, ch) > budget:
        lams = sorted({(cost[i, j] - cost[i, k]) / (bits[i, k] - bits[i, j])
                       for i in range(n) for j in range(m) for k in range(m)
                       if bits[i, k] > bits[i, j] and cost[i, j] > cost[i, k]})
        fit = [lam for lam in lams if _used(bits, _pick(bits, cost, lam)) <= budget]
        if fit:
            ch = _pick(bits, cost, fit[0])
        else:
            # rounding at the largest breakpoint kept a tie on the wider side: take the
            # limit of large lambda, fewest bits (ties: lower cost, then lower index)
            ch = [min(range(m), key=lambda j: (bits[i, j], cost[i, j], j)) for i in range(n)]
    used = _used(bits, ch)
    while True:
        best = None
        for i in range(n):
            b0, c0 = bits[i, ch[i]], cost[i, ch[i]]
            for k in range(m):
                db, dc = bits[i, k] - b0, c0 - cost[i, k]
                if db <= 0.0 or dc <= 0.0 or used + db > budget:
                    continue
                r = dc / db
                if best is None or r > best[0]:
                    best = (r, i, k)
        if best is None:
            return ch
        _, i, k = best
        used += bits[i, k] - bits[i, ch[i]]
        ch[i] = k
