"""Global rank allocation: a plain, literal greedy allocator.

TEST INFRASTRUCTURE ONLY (see the package header).

TraceKV (abstract; ai4snews Synopsis and Interpretation) allocates ranks globally: the limited
rank budget goes to the KV states and singular components that matter most, instead of one rank
per layer. The pages name the step but not its rule. The plainest reading, used here:

  * every matrix m (K or V of a layer) has a spectrum sigma_m[0] >= sigma_m[1] >= ... (the
    singular values of its sensitivity-weighted SVD);
  * keeping rank r of matrix m preserves the energy sum_{k<r} sigma_m[k]^2;
  * ranks start at r_min and grow in granules of g (the storage granularity) up to r_max;
  * while the budget allows another granule, the granule with the largest marginal gain
    sum_{k=r_m}^{r_m+g-1} sigma_m[k]^2 is added (equal gains: the lower matrix index first).

Gains are evaluated in float64, summing the squares of the float32 spectrum in index order (each
square is exact in float64, so the sum's rounding is fixed by that order).

Pins (tests/test_rankalloc_oracle.py): optimality against brute-force enumeration of every
allocation on small problems (for non-increasing spectra the per-matrix energy is concave, so
greedy maximises the total); the budget is used in full when feasible; flat spectra fill the
lowest matrices first; a single matrix takes min(budget, r_max); scaling every spectrum by one
factor changes nothing; an all-zero spectrum stays at r_min.

The rule itself is a reading (the pages do not define the allocator), so the rule's parity with
the pages is unpinned; the oracle is pinned to the rule's own properties above.
"""
from __future__ import annotations

import itertools

import numpy as np


def granule_gain(sigma_row, r: int, g: int) -> float:
    """sum_{k=r}^{r+g-1} sigma[k]^2 in float64, index order."""
    acc = 0.0
    for k in range(r, r + g):
        s = float(np.float32(sigma_row[k]))
        acc = acc + s * s
    return acc


def allocate(sigma, budget: int, r_min: int, r_max: int, g: int) -> np.ndarray:
    """sigma [M, n] (non-increasing rows); returns int ranks [M]."""
    sigma = np.asarray(sigma, np.float32)
    M = sigma.shape[0]
    ranks = [r_min] * M
    left = budget - M * r_min
    if left < 0:
        raise ValueError("budget below M * r_min")
    while left >= g:
        best, best_m = -1.0, -1
        for m in range(M):
            if ranks[m] + g <= r_max:
                gain = granule_gain(sigma[m], ranks[m], g)
                if gain > best:
                    best, best_m = gain, m
        if best_m < 0:
            break
        ranks[best_m] += g
        left -= g
    return np.asarray(ranks, np.int32)


def captured_energy(sigma, ranks) -> float:
    sigma = np.asarray(sigma, np.float64)
    return float(sum(np.sum(sigma[m, :r] ** 2) for m, r in enumerate(ranks)))


def bruteforce_best_energy(sigma, budget: int, r_min: int, r_max: int, g: int) -> float:
    """Max captured energy over every allocation with sum <= budget (tiny problems)."""
    M = np.asarray(sigma).shape[0]
    choices = range(r_min, r_max + 1, g)
    best = -1.0
    for rs in itertools.product(choices, repeat=M):
        if sum(rs) <= budget:
            best = max(best, captured_energy(sigma, rs))
    return best
