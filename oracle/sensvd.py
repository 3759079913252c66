"""Sensitivity-weighted SVD basis construction: plain float64 definitions.

TEST INFRASTRUCTURE ONLY (see the package header).

TraceKV (abstract; ai4snews Synopsis and Interpretation): before the SVD, each KV state is
weighted by its sensitivity (how much a perturbation of it moves the policy), so the limited rank
goes to the states that matter; plain SVD weights all states equally. Reading used here: for the
KV samples x_n (rows of X [N, D]) with sensitivities w_n >= 0, the basis is the top-r right
singular vectors of diag(sqrt(w)) X, i.e. the minimiser of sum_n w_n ||x_n - x_n B^T B||^2 over
bases with orthonormal rows, and the spectrum (its singular values) feeds rank allocation.

Precision reading: the weighted rows y_n = sqrt(w_n) x_n are formed in float32 and rounded once to
bfloat16 (the matrix-core operand), X being bfloat16 already; everything after that is exact
arithmetic on those y_n here (float64).

Functions
---------
``weighted_rows``   y_n = bf16(f32(sqrt(f32(w_n))) * x_n)                [N, D] float64
``gram``            G = Y^T Y                                            [D, D]
``basis``           (B [r, D], sigma [D]): top-r right singular vectors of Y as rows (sign: the
                    largest-magnitude component of each row positive), all singular values
                    descending.

Pins (tests/test_sensvd_oracle.py): orthogonal columns with known norms give those norms as
singular values and unit vectors as the basis; unit weights reduce to the plain SVD of X; an
integer weight equals repeating the sample; scaling all weights by c scales sigma by sqrt(c) and
leaves the basis; rank-1 data gives its direction; the basis beats random orthonormal bases on
the weighted reconstruction error (Eckart-Young); zero-weight samples have no influence.
"""
from __future__ import annotations

import numpy as np

from .append import bf16_rne


def weighted_rows(x, w) -> np.ndarray:
    x32 = np.asarray(x, np.float32)
    sw = np.sqrt(np.asarray(w, np.float32)).astype(np.float32)
    return bf16_rne((sw[:, None] * x32).astype(np.float32)).astype(np.float64)


def gram(x, w) -> np.ndarray:
    y = weighted_rows(x, w)
    return y.T @ y


def _fix_signs(rows: np.ndarray) -> np.ndarray:
    out = rows.copy()
    for i in range(out.shape[0]):
        k = int(np.argmax(np.abs(out[i])))
        if out[i, k] < 0:
            out[i] = -out[i]
    return out


def basis(x, w, r: int):
    """Top-r right singular vectors of Y as rows, and all singular values (descending)."""
    y = weighted_rows(x, w)
    D = y.shape[1]
    if y.shape[0] == 0:
        return np.eye(D)[:r], np.zeros(D)
    # the thin factorisation already holds all D right singular vectors when N >= D
    _, s, vt = np.linalg.svd(y, full_matrices=y.shape[0] < D)
    sig = np.zeros(D)
    sig[:s.shape[0]] = s
    return _fix_signs(vt[:r]), sig


def weighted_error(x, w, b) -> float:
    """sum_n w_n ||x_n - x_n B^T B||^2 (float64, unrounded weights)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    b = np.asarray(b, np.float64)
    res = x - x @ b.T @ b
    return float(np.sum(w * np.sum(res * res, axis=1)))
