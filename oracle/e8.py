"""Nearest point of the E8 lattice (oracle).

[ABS] / [NEWS]: weights are placed, row-normalised, on the E8 lattice (a
uniformly arranged high-dimensional grid) before entropy coding.  The pages do
not give the quantiser; we use the classical decoder of Conway & Sloane,
"Fast quantizing and decoding algorithms for lattice quantizers and codes"
(IEEE Trans. IT, 1982): E8 = D8 u (D8 + 1/2), and the nearest D8 point is the
coordinate-wise rounding, with the worst-rounded coordinate rounded the other
way when the coordinate sum is odd.

Tie-breaking (pages silent; ours, deterministic): rint is round-half-even; the
worst coordinate is the first index of max |v - f|; it moves by +1 when
v - f >= 0, else -1; squared distances are float64 sums taken left to right;
the half-integer coset wins only when strictly closer.

Output is in *doubled* coordinates u = 2p (integers, all of one parity, sum
divisible by 4), so both cosets stay integral.

Pins (tests): brute force over all lattice points near y on tiny inputs, E8
membership, translation by 2Z^8, sign symmetry off ties, and the E8
normalised second moment 929/12960 (Conway & Sloane, SPLAG) by Monte Carlo.
"""
from __future__ import annotations

import numpy as np


def d8_nearest(v: np.ndarray) -> np.ndarray:
    """Nearest D8 point (integer vectors with even sum) to each row of v (n, 8)."""
    v = np.asarray(v, dtype=np.float64)
    f = np.rint(v)
    odd = np.mod(f.sum(axis=1), 2.0) != 0.0
    if odd.any():
        err = v - f
        i = np.argmax(np.abs(err), axis=1)       # first index of the maximum
        rows = np.nonzero(odd)[0]
        ii = i[rows]
        step = np.where(err[rows, ii] >= 0.0, 1.0, -1.0)
        f[rows, ii] += step
    return f


def sq_dist(y: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Sum over the 8 coordinates of (y - p)^2, accumulated left to right in float64."""
    d = (y[:, 0] - p[:, 0]) ** 2
    for i in range(1, 8):
        d = d + (y[:, i] - p[:, i]) ** 2
    return d


def e8_nearest_doubled(y: np.ndarray) -> np.ndarray:
    """Doubled coordinates u = 2 Q_E8(y) (int64, shape (n, 8))."""
    y = np.asarray(y, dtype=np.float64)
    p0 = d8_nearest(y)
    p1 = d8_nearest(y - 0.5) + 0.5
    d0 = sq_dist(y, p0)
    d1 = sq_dist(y, p1)
    pick1 = d1 < d0
    p = np.where(pick1[:, None], p1, p0)
    return (2.0 * p).astype(np.int64)


def is_e8_doubled(u: np.ndarray) -> np.ndarray:
    """Membership test for doubled coordinates: one parity for all 8, sum = 0 mod 4."""
    u = np.asarray(u, dtype=np.int64)
    par = np.mod(u, 2)
    same = (par == par[:, :1]).all(axis=1)
    return same & (np.mod(u.sum(axis=1), 4) == 0)
