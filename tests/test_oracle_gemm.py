"""Pins for the GEMM oracle (oracle.gemm): every output of linear_ref and
linear_fp8_ref against an exactly rounded pure-Python dot product (math.fsum over the
float64 products), on shapes whose three sizes all differ, so that a transposed
operand, a bias or scale on the wrong axis, or a dropped term fails."""
import math

import numpy as np
import pytest

from oracle import numerics as nx
from oracle.gemm import linear_fp8_ref, linear_ref, rel_l2


def _fsum_linear(x, w, bias=None):
    T, K = len(x), len(x[0])
    N = len(w)
    out = []
    for t in range(T):
        row = []
        for n in range(N):
            assert len(w[n]) == K
            terms = [float(x[t][k]) * float(w[n][k]) for k in range(K)]
            if bias is not None:
                terms.append(float(bias[n]))
            row.append(math.fsum(terms))
        out.append(row)
    return out


@pytest.mark.parametrize("T,N,K,with_bias", [(3, 5, 7, True), (4, 2, 9, False), (1, 6, 16, True), (5, 1, 3, True)])
def test_linear_ref_against_fsum(T, N, K, with_bias):
    rng = np.random.default_rng(T * 100 + N * 10 + K)
    # small integers times powers of two: every product and partial sum is exact in
    # float64, so the matmul must equal the exactly rounded sums bit for bit
    x = rng.integers(-64, 65, (T, K)) * 2.0 ** rng.integers(-6, 3, (T, K))
    w = rng.integers(-64, 65, (N, K)) * 2.0 ** rng.integers(-6, 3, (N, K))
    b = rng.integers(-50, 51, N) * 0.25 if with_bias else None
    got = linear_ref(x, w, b)
    ref = np.array(_fsum_linear(x.tolist(), w.tolist(), None if b is None else b.tolist()))
    assert got.shape == (T, N)
    assert np.array_equal(got, ref)


def test_linear_ref_general_values():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 11))
    w = rng.standard_normal((4, 11))
    b = rng.standard_normal(4)
    got = linear_ref(x, w, b)
    ref = np.array(_fsum_linear(x.tolist(), w.tolist(), b.tolist()))
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


def test_linear_fp8_ref_against_fsum():
    rng = np.random.default_rng(11)
    T, N, K = 3, 5, 16
    xq = rng.integers(0, 256, (T, K)).astype(np.uint8)
    wq = rng.integers(0, 256, (N, K)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x38        # E4M3FN has no infinity; 0x7F/0xFF are NaN
    wq[(wq & 0x7F) == 0x7F] = 0x30
    xf, wf = nx.fp8_e4m3fn_to_f64(xq), nx.fp8_e4m3fn_to_f64(wq)
    a_x = 0.375
    a_r = np.array([0.5, 2.0, 0.125, 3.0, 1.0])          # non-uniform per output row
    got = linear_fp8_ref(xf, wf, a_x, a_r)
    plain = np.array(_fsum_linear(xf.tolist(), wf.tolist()))
    ref = np.array([[plain[t][n] * a_x * a_r[n] for n in range(N)] for t in range(T)])
    assert got.shape == (T, N)
    assert np.allclose(got, ref, rtol=1e-15, atol=0)
    # the per-row scale belongs to the output column: swapping it onto the tokens fails
    assert not np.allclose(plain * a_x * a_r[:T, None], ref)


def test_rel_l2():
    assert rel_l2([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert rel_l2([0.0, 0.0], [3.0, 4.0]) == 1.0
    assert math.isclose(rel_l2([3.0, 4.5], [3.0, 4.0]), 0.1)
