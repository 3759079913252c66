"""Historical-coordinate sync after a basis update: plain float64 definitions.

TEST INFRASTRUCTURE ONLY (see the package header).

iS-KV ("iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD", English
abstract; method summary, 技术框架 and 关键创新): the low-rank basis evolves while decoding,
and the coordinates of the stored history are synchronised with the updated basis; without the
sync, old coordinates read in the new basis describe a drifted history.

The pages name the sync, not its formula. The plainest reading: each stored latent row z (a
token whose reconstruction is z B) is replaced by its least-squares coordinates in the new
basis B' [r', D]:

    z' = argmin_y || y B' - z B ||  =  z B pinv(B')  =  z W^T,     W = (B pinv(B'))^T  [r', r]

W is computed by the caller (as the down-projection P of the append path is) and handed to the
library in the base dtype; the library only applies it. Storage of z' follows the append path:
float32 caches keep f32(z'), bf16 caches keep bf16_rne(f32(z')).

Pins (tests/test_rebase_oracle.py): B' = B gives W = I and z' = z; B' = R B with R invertible
(same row space) gives z' B' = z B; for a general B', z' B' is the orthogonal projection of z B
onto the row space of B'; the stale coordinates (no sync) reconstruct z B' != z B; and the
row-by-row definition equals brute force on tiny shapes.
"""
from __future__ import annotations

import numpy as np

from .append import bf16_rne


def sync_weights(b_old, b_new) -> np.ndarray:
    """W = (B pinv(B'))^T [r', r]: row j holds the old coordinates' weights of new index j."""
    b_old = np.asarray(b_old, np.float64)
    b_new = np.asarray(b_new, np.float64)
    return (b_old @ np.linalg.pinv(b_new)).T


def rebase_rows(z, w) -> np.ndarray:
    """z' = z W^T for stored rows z [n, r] and W [r', r], in float64."""
    return np.asarray(z, np.float64) @ np.asarray(w, np.float64).T


def rebase_bruteforce(z, w) -> list:
    """The same sums with Python loops (tiny shapes)."""
    z = [[float(x) for x in row] for row in np.asarray(z)]
    w = [[float(x) for x in row] for row in np.asarray(w)]
    return [[sum(zi * wj[i] for i, zi in enumerate(row)) for wj in w] for row in z]


def store(z64, latent: str) -> np.ndarray:
    """Storage form of float64 rows: float32, or bf16 (round to nearest even) held in float32."""
    z32 = np.asarray(z64, np.float64).astype(np.float32)
    if latent == "f32":
        return z32
    if latent == "bf16":
        return bf16_rne(z32)
    raise ValueError(latent)
