"""Pins for the oracle's symbol model: frequency quantiser invariants, the
magnitude symbol bijection, LAST restriction vs E8 parity, table sums and the
fixed-point log table."""
import math

import numpy as np
import pytest

from oracle import model as mdl
from oracle.e8 import e8_nearest_doubled


@pytest.mark.parametrize("seed", range(6))
def test_quantize_freqs_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 300))
    w = rng.integers(0, 10 ** rng.integers(1, 9), size=n)
    w[rng.random(n) < 0.3] = 0
    ids = np.arange(n)
    for T in (1024, 2048):
        f = mdl.quantize_freqs(w, ids, T)
        assert f.sum() == T
        assert (f[w > 0] >= 1).all()
        assert ((f > 0).sum() >= 2)
        assert f.max() <= T - 1
        # idempotent: quantising a table that already sums to T returns it
        assert np.array_equal(mdl.quantize_freqs(f, ids, T), f)
        # monotone in the weight: larger weight never gets a smaller frequency
        order = np.argsort(w, kind="stable")
        present = f[order][w[order] > 0]
        assert (np.diff(present) >= -1).all()


def test_quantize_freqs_degenerate():
    f = mdl.quantize_freqs([0, 5, 0, 0], [0, 1, 2, 3], 2048)
    assert list(f) == [1, 2047, 0, 0]
    f = mdl.quantize_freqs([0, 0, 0], [0, 1, 2], 1024)
    assert list(f) == [512, 512, 0]


@pytest.mark.parametrize("k", [3, 4, 5, 6, 7])
def test_magnitude_symbol_bijection(k):
    rng = np.random.default_rng(k)
    m = np.concatenate([np.arange(0, 1 << 16), rng.integers(0, 1 << 29, size=200000),
                        (1 << np.arange(0, 29)), (1 << np.arange(1, 30)) - 1])
    msym, raw, rb = mdl.magnitude_symbol(m, k)
    assert (msym < mdl.n_msym(k)).all()
    assert (raw < (np.int64(1) << rb)).all()
    assert np.array_equal(mdl.magnitude_from_symbol(msym, raw, k), m)
    # buckets are monotone in m
    o = np.argsort(m)
    assert (np.diff(msym[o]) >= 0).all()
    # direct symbols below K carry no raw bits
    assert (rb[m < (1 << k)] == 0).all()


@pytest.mark.parametrize("scale", [0.3, 3.0, 40.0, 3000.0])
def test_last_restriction_matches_e8_parity(scale):
    rng = np.random.default_rng(7)
    u = e8_nearest_doubled(rng.standard_normal((20000, 8)) * scale)
    for k in (3, 5, 7):
        sym = mdl.group_symbols(u, k)     # asserts the implied LSB of last-coordinate buckets
        counts = mdl.count_symbols(sym, mdl.n_msym(k))
        m = mdl.build_model(k, *counts)
        for c in (0, 1):
            for pi in (0, 1):
                sel = (sym["c"] == c) & (sym["pi"] == pi)
                alph = set(m.last_alphabet(c, pi).tolist())
                assert set(sym["id"][sel, 7].tolist()) <= alph
        # every coded symbol has a nonzero frequency in its table
        assert (m.F[sym["ctx"], sym["id"]] > 0).all()


@pytest.mark.parametrize("k,P", [(4, 10), (5, 10), (6, 11), (7, 11)])
def test_tables_sum_and_roundtrip(k, P):
    rng = np.random.default_rng(9)
    u = e8_nearest_doubled(rng.standard_normal((5000, 8)) * 5.0 * (1 << (k - 4)))
    sym = mdl.group_symbols(u, k)
    m = mdl.build_model(k, *mdl.count_symbols(sym, mdl.n_msym(k)))
    assert m.P == P == mdl.precision(k) and m.M == 1 << P
    assert (m.F.sum(axis=1) == m.M).all()
    assert m.F.max() <= m.M - 1
    # FREE: signs split a magnitude's probability evenly
    for c in (0, 1):
        f = m.F[1 + c, :2 * m.nm]
        assert np.array_equal(f[2::2], f[3::2])
    m2 = mdl.Model.from_bytes(m.to_bytes(), k)
    assert np.array_equal(m2.F, m.F)


def test_log2q_clear_of_ties():
    t = mdl.LOG2Q
    for f in range(1, mdl.M_MAX + 1):
        x = 65536.0 * math.log2(f)
        assert abs((x - math.floor(x)) - 0.5) > 1e-6
    for j in range(12):
        assert t[1 << j] == 65536 * j
