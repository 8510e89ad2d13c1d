"""Pins of the budgeted-bitrate oracle: brute force over every combination, the
FP32-container decode, the E8 second moment."""
import itertools
import math

import numpy as np
import pytest

import synth
import oracle
from oracle import numerics as nx, plan


def _brute(bits, cost, budget):
    n, m = bits.shape
    best = None
    for ch in itertools.product(range(m), repeat=n):
        b = sum(bits[i, j] for i, j in enumerate(ch))
        if b <= budget:
            c = sum(cost[i, j] for i, j in enumerate(ch))
            best = c if best is None or c < best else best
    return best


def _instance(rng, n, m):
    # rate-distortion-like candidates: bits grow, cost mostly falls (not always convex)
    bits = np.sort(rng.uniform(1.0, 10.0, size=(n, m)), axis=1) * rng.integers(100, 1000, size=(n, 1))
    cost = np.sort(rng.uniform(0.01, 5.0, size=(n, m)), axis=1)[:, ::-1].copy()
    cost[rng.random((n, m)) < 0.1] *= 3.0
    return bits, cost


@pytest.mark.parametrize("seed", range(12))
def test_plan_optimal_at_lagrangian_budgets(seed):
    rng = np.random.default_rng(seed)
    n, m = int(rng.integers(2, 5)), int(rng.integers(2, 5))
    bits, cost = _instance(rng, n, m)
    lams = sorted({(cost[i, j] - cost[i, k]) / (bits[i, k] - bits[i, j])
                   for i in range(n) for j in range(m) for k in range(m)
                   if bits[i, k] > bits[i, j] and cost[i, j] > cost[i, k]}) + [0.0]
    for lam in lams:
        ch = plan._pick(bits, cost, lam)
        budget = plan._used(bits, ch)
        got = plan.plan(bits, cost, budget)
        c_got = sum(cost[i, j] for i, j in enumerate(got))
        assert plan._used(bits, got) <= budget
        assert math.isclose(c_got, _brute(bits, cost, budget), rel_tol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_plan_within_duality_gap(seed):
    # Between Lagrangian budgets: feasible, no worse than its Lagrangian start
    # (upgrades only lower the cost), and above the brute-force optimum by at
    # most lambda * (budget - bits of the start), the duality-gap bound.
    rng = np.random.default_rng(100 + seed)
    n, m = int(rng.integers(1, 6)), int(rng.integers(1, 5))
    bits, cost = _instance(rng, n, m)
    lams = sorted({(cost[i, j] - cost[i, k]) / (bits[i, k] - bits[i, j])
                   for i in range(n) for j in range(m) for k in range(m)
                   if bits[i, k] > bits[i, j] and cost[i, j] > cost[i, k]})
    lo, hi = float(bits.min(axis=1).sum()), float(bits.max(axis=1).sum())
    for budget in list(np.linspace(lo, hi, 9)) + [float(bits[:, q].sum()) for q in range(m)]:
        got = plan.plan(bits, cost, budget)
        c_got = sum(cost[i, j] for i, j in enumerate(got))
        assert plan._used(bits, got) <= budget
        lam = 0.0
        if plan._used(bits, plan._pick(bits, cost, 0.0)) > budget:
            fit = [l for l in lams if plan._used(bits, plan._pick(bits, cost, l)) <= budget]
            lam = fit[0] if fit else lams[-1]
        start = plan._pick(bits, cost, lam)
        if plan._used(bits, start) > budget:     # tie rounded to the wider side
            start = [int(np.lexsort((cost[i], bits[i]))[0]) for i in range(n)]
        c_start = sum(cost[i, j] for i, j in enumerate(start))
        opt = _brute(bits, cost, budget)
        assert opt <= c_got * (1 + 1e-12) and c_got <= c_start * (1 + 1e-12)
        assert c_got - opt <= lam * (budget - plan._used(bits, start)) * (1 + 1e-9) + 1e-12
    with pytest.raises(plan.Infeasible):
        plan.plan(bits, cost, lo * 0.999)


def test_distortion_matches_fp32_decode_and_theory():
    src = synth.rowscaled_f32(96, 256, 31)
    for t in (3.0, 6.0):
        blob = oracle.compress(src, nx.DT_FP32, t)
        e, r = plan.distortion(src, nx.DT_FP32, blob)
        _, out, _ = oracle.decode(blob)
        d = src.astype(np.float64) - out.astype(np.float64)
        assert math.isclose(e, float(np.sum(d * d)), rel_tol=1e-12)
        assert math.isclose(r, float(np.sum(src.astype(np.float64) ** 2)), rel_tol=1e-12)
    # high rate: mean squared error per coordinate = (2 delta)^2 G(E8) h-weighted; in
    # relative terms rel^2 ~ 4 G delta^2 when rows are RMS-normalised
    b = oracle.parse_blob(blob)
    rel2 = e / r
    G = 929.0 / 12960.0
    assert abs(rel2 / (4.0 * G * float(b.delta) ** 2) - 1.0) < 0.1
