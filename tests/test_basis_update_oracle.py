"""Pins of the block-incremental basis update oracle (oracle/basis_update.py).

The oracle follows Brand's steps (project, residual QR, core SVD, rotate, truncate); the pins hold
it to what the mathematics fixes independently of those steps: the batch SVD of the whole stacked
history (numpy's SVD of the full-size rows, not of the small core), span invariance, Eckart-Young
and the orthogonal-projection property of the coordinate sync. A copy with a planted slip fails.
"""
import numpy as np
import pytest

from oracle import basis_update as BU


def _orthonormal_rows(rng, r, D):
    q, rr = np.linalg.qr(rng.standard_normal((D, r)))
    return (q * np.sign(np.diag(rr))[None, :]).T


def _history(rng, T, r, D, decay=0.7):
    """X = U diag(sigma) B exactly: T rows of rank r with a gapped spectrum."""
    B = _orthonormal_rows(rng, r, D)
    U = _orthonormal_rows(rng, r, T).T                 # [T, r] orthonormal columns
    sigma = 10.0 * decay ** np.arange(r)
    return U @ np.diag(sigma) @ B, sigma, B


def _same_rows_up_to_sign(a, b, atol):
    assert a.shape == b.shape
    for i in range(a.shape[0]):
        d = min(np.max(np.abs(a[i] - b[i])), np.max(np.abs(a[i] + b[i])))
        assert d <= atol, (i, d)


@pytest.mark.parametrize("T,r,n,D", [(50, 6, 3, 16), (300, 20, 8, 64), (40, 4, 12, 32)])
def test_no_truncation_equals_the_batch_svd_of_all_rows(T, r, n, D):
    rng = np.random.default_rng(T + r)
    X, sigma, B = _history(rng, T, r, D)
    Y = rng.standard_normal((n, D))
    Bn, sn = BU.incremental_update(sigma, B, Y, r + n)
    _, s_all, vt_all = np.linalg.svd(np.concatenate([X, Y], axis=0), full_matrices=False)
    np.testing.assert_allclose(sn, s_all[:r + n], rtol=1e-10, atol=1e-10)
    _same_rows_up_to_sign(Bn, vt_all[:r + n], 1e-8)
    # sign convention: each row's largest-magnitude component is positive
    assert np.all(Bn[np.arange(r + n), np.argmax(np.abs(Bn), axis=1)] > 0)
    # orthonormal rows
    np.testing.assert_allclose(Bn @ Bn.T, np.eye(r + n), atol=1e-10)


def test_truncated_update_equals_truncated_batch_svd():
    rng = np.random.default_rng(5)
    X, sigma, B = _history(rng, 200, 16, 64)
    Y = 3.0 * rng.standard_normal((10, 64))
    Bn, sn = BU.incremental_update(sigma, B, Y, 16)
    _, s_all, vt_all = np.linalg.svd(np.concatenate([X, Y], axis=0), full_matrices=False)
    np.testing.assert_allclose(sn, s_all[:16], rtol=1e-10)
    _same_rows_up_to_sign(Bn, vt_all[:16], 1e-8)


def test_rows_inside_the_span_leave_the_span_unchanged():
    rng = np.random.default_rng(6)
    _, sigma, B = _history(rng, 100, 12, 48)
    Y = rng.standard_normal((7, 12)) @ B                 # new rows in span(B)
    Bn, sn = BU.incremental_update(sigma, B, Y, 12)
    np.testing.assert_allclose(Bn.T @ Bn, B.T @ B, atol=1e-10)
    # the new spectrum is that of diag(sigma) stacked with the coordinates C = Y B^T
    C = Y @ B.T
    s_ref = np.linalg.svd(np.concatenate([np.diag(sigma), C], axis=0), compute_uv=False)
    np.testing.assert_allclose(sn, s_ref, rtol=1e-10)


def test_eckart_young():
    rng = np.random.default_rng(7)
    X, sigma, B = _history(rng, 120, 10, 40)
    Y = rng.standard_normal((9, 40))
    M = np.concatenate([np.diag(sigma) @ B, Y], axis=0)
    for r_new in (1, 5, 10, 15):
        Bn, _ = BU.incremental_update(sigma, B, Y, r_new)
        best = np.linalg.norm(M - M @ Bn.T @ Bn) ** 2
        s_full = np.linalg.svd(M, compute_uv=False)
        np.testing.assert_allclose(best, np.sum(s_full[r_new:] ** 2), rtol=1e-9, atol=1e-9)
        for _ in range(5):
            Q = _orthonormal_rows(rng, r_new, 40)
            assert np.linalg.norm(M - M @ Q.T @ Q) ** 2 >= best - 1e-9
        # a perturbed optimum is worse too
        P = Bn + 1e-3 * rng.standard_normal(Bn.shape)
        P = np.linalg.qr(P.T)[0].T
        assert np.linalg.norm(M - M @ P.T @ P) ** 2 >= best - 1e-12


def test_sync_is_the_orthogonal_projection_onto_the_new_basis():
    rng = np.random.default_rng(8)
    X, sigma, B = _history(rng, 60, 8, 32)
    Y = rng.standard_normal((5, 32))
    Bn, _ = BU.incremental_update(sigma, B, Y, 10)
    W = BU.sync_weights(B, Bn)
    assert W.shape == (10, 8)
    z = X @ B.T                                          # stored coordinates of the history
    z_new = z @ W.T
    np.testing.assert_allclose(z_new @ Bn, (z @ B) @ Bn.T @ Bn, atol=1e-10)
    # residual orthogonal to the new row space
    res = z @ B - z_new @ Bn
    np.testing.assert_allclose(res @ Bn.T, 0.0, atol=1e-10)
    # update by rows inside span(B) at the same rank: the history is reproduced exactly
    Bs, _ = BU.incremental_update(sigma, B, rng.standard_normal((4, 8)) @ B, 8)
    np.testing.assert_allclose((z @ BU.sync_weights(B, Bs).T) @ Bs, X, atol=1e-9)


def test_empty_history_spectrum_is_the_svd_of_the_block():
    rng = np.random.default_rng(9)
    B = _orthonormal_rows(rng, 3, 20)
    Y = rng.standard_normal((6, 20))
    Bn, sn = BU.incremental_update(np.zeros(3), B, Y, 6)
    _, s, vt = np.linalg.svd(Y, full_matrices=False)
    np.testing.assert_allclose(sn, s, rtol=1e-10)
    _same_rows_up_to_sign(Bn, vt, 1e-8)


def test_rank_out_of_range_is_rejected():
    B = np.eye(4, 8)
    with pytest.raises(ValueError):
        BU.incremental_update(np.ones(4), B, np.ones((2, 8)), 7)
    with pytest.raises(ValueError):
        BU.incremental_update(np.ones(4), B, np.ones((2, 8)), 0)


def _slipped(kind):
    """Copies of the update with one plausible mistake each (planted on the CPU only)."""
    def f(sigma, basis, rows, rank_new):
        s = np.asarray(sigma, np.float64)
        B = np.asarray(basis, np.float64)
        Y = np.asarray(rows, np.float64)
        r, D = B.shape
        n = Y.shape[0]
        C = Y @ B.T
        R = Y - C @ B if kind != "no_projection" else Y
        Q, T = np.linalg.qr(R.T)
        Kc = np.zeros((r + n, r + n))
        Kc[:r, :r] = np.diag(s) if kind != "unweighted" else np.eye(r)
        Kc[r:, :r] = C
        Kc[r:, r:] = T.T if kind != "untransposed_T" else T
        _, sv, Vt = np.linalg.svd(Kc)
        Bn = Vt @ np.concatenate([B, Q.T], axis=0)
        return BU.sign_fix(Bn[:rank_new]), sv[:rank_new]
    return f


@pytest.mark.parametrize("kind", ["unweighted", "no_projection", "untransposed_T"])
def test_planted_slips_fail_the_batch_pin(kind):
    rng = np.random.default_rng(10)
    X, sigma, B = _history(rng, 80, 6, 24)
    Y = rng.standard_normal((4, 24))
    _, s_all, _ = np.linalg.svd(np.concatenate([X, Y], axis=0), full_matrices=False)
    _, sn = _slipped(kind)(sigma, B, Y, 10)
    assert np.max(np.abs(sn - s_all[:10])) > 1e-3
