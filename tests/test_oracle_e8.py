"""Pins for the oracle's E8 quantiser: brute force, membership, invariances,
kissing number, covering radius and the E8 second moment (SPLAG)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.e8 import e8_nearest_doubled, is_e8_doubled

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e8_facts.json")))


def _brute_nearest_dist2(y):
    """Exhaustive nearest E8 point near y: both cosets, every coordinate within +-1 of the
    rounded value, even-sum filter.  Distances by a dot product (not the oracle's sum)."""
    best = np.inf
    for half in (0.0, 0.5):
        base = np.floor(y - half)
        cands = [np.array([b - 1, b, b + 1, b + 2]) for b in base]
        grid = np.array(list(itertools.product(*cands)))          # (4^8, 8)
        grid = grid[np.mod(grid.sum(axis=1), 2) == 0] + half
        d = grid - y
        best = min(best, float(np.min(np.einsum("ij,ij->i", d, d))))
    return best


def test_brute_force_random():
    rng = np.random.default_rng(11)
    y = rng.uniform(-3, 3, size=(40, 8))
    u = e8_nearest_doubled(y)
    for i in range(len(y)):
        d = y[i] - u[i] / 2.0
        assert abs(float(d @ d) - _brute_nearest_dist2(y[i])) <= 1e-12


def test_brute_force_ties():
    # points on Voronoi boundaries: half-integers, deep holes, midpoints of minimal vectors
    ys = [np.zeros(8), np.full(8, 0.25), np.eye(8)[0], np.full(8, 0.5) * np.array([1, 1, 1, 1, 0, 0, 0, 0]),
          np.array([0.5, 0.5, 0, 0, 0, 0, 0, 0]), np.array([1.0, 0, 0, 0, 0, 0, 0, 0]) * 2.5,
          np.array([0.75, 0.25, 0.25, 0.25, 0.25, 0.25, 0.25, 0.25]), np.full(8, -0.25)]
    y = np.array(ys)
    u = e8_nearest_doubled(y)
    assert is_e8_doubled(u).all()
    for i in range(len(y)):
        d = y[i] - u[i] / 2.0
        assert abs(float(d @ d) - _brute_nearest_dist2(y[i])) <= 1e-12
    # deterministic
    assert np.array_equal(u, e8_nearest_doubled(y))


def test_membership_large_scale():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((20000, 8)) * 1000.0
    u = e8_nearest_doubled(y)
    assert is_e8_doubled(u).all()
    # nearest point is within the covering radius
    d = y - u / 2.0
    assert (np.einsum("ij,ij->i", d, d) <= GOLD["covering_radius_sq"] + 1e-9).all()


def test_translation_and_sign():
    rng = np.random.default_rng(2)
    y = np.round(rng.uniform(-4, 4, size=(5000, 8)) * 2 ** 20) / 2 ** 20
    z = rng.integers(-5, 6, size=(5000, 8))
    u = e8_nearest_doubled(y)
    assert np.array_equal(e8_nearest_doubled(y + 2 * z), u + 4 * z)
    assert np.array_equal(e8_nearest_doubled(-y), -u)


def test_kissing_number_and_fixed_points():
    # all doubled vectors with sum of squares 8 (norm 2) that are E8 points
    vals = [-2, -1, 0, 1, 2]
    pts = np.array([p for p in itertools.product(vals, repeat=8) if sum(v * v for v in p) == 8])
    pts = pts[is_e8_doubled(pts)]
    assert len(pts) == GOLD["kissing_number"]
    # lattice points are their own nearest point
    assert np.array_equal(e8_nearest_doubled(pts / 2.0), pts)


def test_second_moment():
    rng = np.random.default_rng(3)
    y = rng.uniform(0.0, 2.0, size=(400000, 8))
    u = e8_nearest_doubled(y)
    d = y - u / 2.0
    g = float(np.mean(np.einsum("ij,ij->i", d, d)) / 8.0)
    expect = GOLD["normalized_second_moment_num"] / GOLD["normalized_second_moment_den"]
    # D8 alone would give 0.0766, Z8 1/12: the tolerance separates them
    assert abs(g - expect) < 6e-4, (g, expect)
