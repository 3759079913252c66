"""Pins of the historical-coordinate sync oracle (oracle/rebase.py) against closed forms."""
import numpy as np
import pytest

from oracle import rebase as RB


def basis(rng, r, D=64):
    q, _ = np.linalg.qr(rng.standard_normal((D, r)))
    return q.T                                   # [r, D], orthonormal rows


def test_same_basis_is_identity():
    rng = np.random.default_rng(1)
    b = basis(rng, 12)
    w = RB.sync_weights(b, b)
    assert np.allclose(w, np.eye(12), atol=1e-12)
    z = rng.standard_normal((9, 12))
    assert np.allclose(RB.rebase_rows(z, w), z, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_same_row_space_keeps_the_reconstruction(seed):
    """B' = R B (R invertible, not orthogonal): the history's reconstruction is unchanged."""
    rng = np.random.default_rng(seed)
    r = 10
    b = basis(rng, r) * rng.uniform(0.5, 2.0, (r, 1))      # not orthonormal either
    R = rng.standard_normal((r, r)) + 3 * np.eye(r)
    b_new = R @ b
    z = rng.standard_normal((7, r))
    z2 = RB.rebase_rows(z, RB.sync_weights(b, b_new))
    assert np.allclose(z2 @ b_new, z @ b, atol=1e-10)
    assert np.allclose(z2, z @ np.linalg.inv(R), atol=1e-10)


@pytest.mark.parametrize("r_new", [4, 10, 16])
def test_general_update_projects_onto_the_new_row_space(r_new):
    rng = np.random.default_rng(r_new)
    D, r = 64, 10
    b = basis(rng, r, D)
    b_new = basis(rng, r_new, D)
    z = rng.standard_normal((5, r))
    z2 = RB.rebase_rows(z, RB.sync_weights(b, b_new))
    proj = b_new.T @ np.linalg.solve(b_new @ b_new.T, b_new)   # projector onto rowspace(B')
    assert np.allclose(z2 @ b_new, (z @ b) @ proj, atol=1e-10)
    # least squares: the residual is orthogonal to the new row space
    resid = z @ b - z2 @ b_new
    assert np.allclose(resid @ b_new.T, 0.0, atol=1e-10)


def test_stale_coordinates_drift_and_the_sync_repairs_them():
    """Reading old coordinates in a rotated basis changes the history; the sync restores it."""
    rng = np.random.default_rng(5)
    r = 8
    b = basis(rng, r)
    theta = 0.3
    rot = np.eye(r)
    rot[:2, :2] = [[np.cos(theta), -np.sin(theta)], [np.sin(theta), np.cos(theta)]]
    b_new = rot @ b                              # same span, rotated coordinates
    z = rng.standard_normal((20, r))
    stale = z @ b_new
    assert np.linalg.norm(stale - z @ b) > 0.1 * np.linalg.norm(z @ b)
    synced = RB.rebase_rows(z, RB.sync_weights(b, b_new)) @ b_new
    assert np.allclose(synced, z @ b, atol=1e-10)


def test_matches_bruteforce():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    assert np.allclose(RB.rebase_rows(z, w), np.array(RB.rebase_bruteforce(z, w)), atol=1e-12)


def test_store_rounds_like_the_append_path():
    z = np.array([[1.0 + 2.0 ** -9, -3.0]])
    assert RB.store(z, "f32").dtype == np.float32
    assert RB.store(z, "bf16")[0, 0] == np.float32(1.0)     # tie to even
    with pytest.raises(ValueError):
        RB.store(z, "i4g32")
