"""Block-incremental basis update of a low-rank KV history (iS-KV).

TEST INFRASTRUCTURE ONLY (see the package header).

iS-KV ("iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD",
English abstract and method summary): the recent window stays exact while older
states are folded, block by block, into a bounded-rank representation whose
low-rank basis is updated incrementally; the stored historical coordinates are
then synchronised with the updated basis. The pages name the technique
(block-incremental SVD) without giving its equations, so this module takes the
textbook one: Brand's incremental SVD ("Incremental singular value decomposition
of uncertain data with missing values", ECCV 2002; "Fast low-rank modifications
of the thin singular value decomposition", 2006), block form.

State of one KV matrix (K or V of one layer): the history rows X [T, D] are kept
as X ~ U diag(sigma) B, with B [r, D] orthonormal rows (the basis the latents are
coordinates in: z_t = x_t B^T) and sigma [r] the singular values. Folding a block
of dense rows Y [n, D] (e.g. the tokens leaving the exact window) means taking the
rank-r' SVD of the stacked rows

    M = [ X ; Y ] = [ U 0 ; 0 I ] [ diag(sigma) B ; Y ]

whose right singular vectors and values are those of the small-left-factor form
M' = [ diag(sigma) B ; Y ] (U has orthonormal columns). Brand's steps, in order:

  1. C = Y B^T                    coordinates of the new rows in the old basis [n, r]
  2. R = Y - C B                  the part of the new rows outside span(B)    [n, D]
  3. R^T = Q T  (thin QR)         Q [D, n] orthonormal, orthogonal to span(B)
  4. Kc = [ diag(sigma)  0 ;      the (r + n) x (r + n) core, with
            C            T^T ]    M' = Kc [ B ; Q^T ]   ([B ; Q^T] orthonormal rows)
  5. Kc = Uk diag(s) Vk^T         SVD of the core
  6. B' = (Vk^T [ B ; Q^T ])[:r'], sigma' = s[:r']

Then the coordinate sync (iS-KV: historical coordinates follow the new basis) is
z' = z B B'^T = z W^T with W = B' B^T [r', r] (B' has orthonormal rows, so
pinv(B') = B'^T), which is the least-squares reading already used for the sync
itself (oracle.rebase).

Sign convention (the same as oracle.sensvd): each basis row has its
largest-magnitude component positive.

Pins (tests/test_basis_update_oracle.py): without truncation (r' = r + n) B' and
sigma' equal numpy's SVD of the whole stacked history [X ; Y] built at full size;
rows inside span(B) leave span(B) unchanged; Eckart-Young (no rank-r' basis does
better, and the residual energy equals the dropped sigma'^2); the sync reproduces
the orthogonal projection of the history onto the new basis; a copy of the
update with a planted slip is caught by the batch pin.
"""
from __future__ import annotations

import numpy as np


def sign_fix(rows: np.ndarray) -> np.ndarray:
    """Each row multiplied by the sign of its largest-magnitude component."""
    rows = np.array(rows, dtype=np.float64, copy=True)
    if rows.size == 0:
        return rows
    idx = np.argmax(np.abs(rows), axis=1)
    s = np.sign(rows[np.arange(rows.shape[0]), idx])
    s[s == 0] = 1.0
    return rows * s[:, None]


def incremental_update(sigma, basis, rows, rank_new: int):
    """Brand's block update of (sigma [r], basis B [r, D]) by the dense rows Y [n, D].

    Returns (B' [rank_new, D], sigma' [rank_new]) in float64: the top rank_new right
    singular vectors (rows, sign-fixed) and singular values of [diag(sigma) B ; Y]."""
    s = np.asarray(sigma, np.float64)
    B = np.asarray(basis, np.float64)
    Y = np.asarray(rows, np.float64)
    r, D = B.shape
    n = Y.shape[0]
    if not 1 <= rank_new <= min(D, r + n):
        raise ValueError("rank_new must be in 1..min(D, r + n)")
    C = Y @ B.T                                   # 1
    R = Y - C @ B                                 # 2
    Q, T = np.linalg.qr(R.T)                      # 3: R^T = Q T, Q [D, n]
    Kc = np.zeros((r + n, r + n))                 # 4
    Kc[:r, :r] = np.diag(s)
    Kc[r:, :r] = C
    Kc[r:, r:] = T.T
    _, sv, Vt = np.linalg.svd(Kc)                 # 5
    Bn = Vt @ np.concatenate([B, Q.T], axis=0)    # 6
    return sign_fix(Bn[:rank_new]), sv[:rank_new]


def sync_weights(basis_old, basis_new) -> np.ndarray:
    """W = B' B^T [r', r]: a stored row z (old coordinates) becomes z' = z W^T."""
    return np.asarray(basis_new, np.float64) @ np.asarray(basis_old, np.float64).T
