"""GEMM oracle for the compressed linear layer.

[README] quick start: a compressed linear layer is called like ``layer(x)`` and
returns what a normal linear layer would.  The definition used:
Y = X W_hat^T (+ bias), evaluated in float64 with NumPy's matmul (a library
primitive), from the BF16 activations and the decoded container weights.
FP8 variant: Y = (X_q W_q^T) * a_x * a_r with per-tensor activation scale a_x
and per-row weight scales a_r ([README] "FP8@5": FP8 W8A8 weight codes, FP8
GEMM at inference).

Pins (tests/test_oracle_gemm.py): every output of both functions equals an
exactly rounded pure-Python dot product (math.fsum over the float64 products) on
shapes whose three sizes all differ, with a bias and a non-uniform per-row scale,
bit for bit where the inputs make every partial sum exact.
"""
from __future__ import annotations

import numpy as np


def linear_ref(x_f64: np.ndarray, w_f64: np.ndarray, bias=None) -> np.ndarray:
    y = np.asarray(x_f64, np.float64) @ np.asarray(w_f64, np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def linear_fp8_ref(xq_f64, wq_f64, a_x: float, a_r) -> np.ndarray:
    y = np.asarray(xq_f64, np.float64) @ np.asarray(wq_f64, np.float64).T
    return y * float(a_x) * np.asarray(a_r, np.float64)[None, :]


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
