"""Pins of the global rank allocation oracle (oracle/rankalloc.py)."""
import numpy as np
import pytest

from oracle import rankalloc as RA


def spectra(rng, M, n, lo=0.3, hi=1.5):
    alpha = rng.uniform(lo, hi, size=M)
    scale = rng.uniform(0.5, 2.0, size=M)
    k = np.arange(1, n + 1, dtype=np.float64)
    return (scale[:, None] * k[None, :] ** (-alpha[:, None] / 2)).astype(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_greedy_is_optimal_against_bruteforce(seed):
    rng = np.random.default_rng(seed)
    M, n, g, r_min, r_max = 3, 16, 2, 2, 12
    s = spectra(rng, M, n)
    budget = int(rng.integers(M * r_min, M * r_max + 1))
    ranks = RA.allocate(s, budget, r_min, r_max, g)
    best = RA.bruteforce_best_energy(s, budget, r_min, r_max, g)
    assert abs(RA.captured_energy(s, ranks) - best) <= 1e-9 * best


def test_budget_is_used_in_full():
    rng = np.random.default_rng(7)
    s = spectra(rng, 10, 64)
    ranks = RA.allocate(s, 10 * 8 + 37 * 4, 8, 64, 4)
    assert ranks.sum() == 10 * 8 + 37 * 4
    assert (ranks % 4 == 0).all() and ranks.min() >= 8 and ranks.max() <= 64


def test_flat_spectra_fill_the_lowest_matrices_first():
    s = np.ones((4, 32), np.float32)
    ranks = RA.allocate(s, 4 * 8 + 3 * 8, 8, 32, 8)
    assert ranks.tolist() == [32, 8, 8, 8]       # equal gains: the lowest matrix, granule by granule


def test_single_matrix_takes_min_of_budget_and_cap():
    s = np.linspace(2, 1, 40, dtype=np.float32)[None]
    assert RA.allocate(s, 24, 8, 40, 8).tolist() == [24]
    assert RA.allocate(s, 400, 8, 40, 8).tolist() == [40]


def test_scaling_all_spectra_changes_nothing():
    rng = np.random.default_rng(3)
    s = spectra(rng, 6, 48)
    a = RA.allocate(s, 6 * 8 + 80, 8, 48, 8)
    b = RA.allocate(s * np.float32(4.0), 6 * 8 + 80, 8, 48, 8)
    np.testing.assert_array_equal(a, b)


def test_zero_spectrum_stays_at_r_min():
    rng = np.random.default_rng(4)
    s = spectra(rng, 5, 32)
    s[2] = 0
    ranks = RA.allocate(s, 5 * 4 + 40, 4, 32, 4)
    assert ranks[2] == 4


def test_budget_below_the_floor_is_rejected():
    with pytest.raises(ValueError):
        RA.allocate(np.ones((3, 8), np.float32), 5, 2, 8, 2)
