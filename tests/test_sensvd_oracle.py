"""Pins of the sensitivity-weighted SVD oracle (oracle/sensvd.py)."""
import numpy as np
import pytest

from oracle import sensvd as SV


def test_orthogonal_columns_give_their_norms():
    rng = np.random.default_rng(0)
    N, D = 64, 16
    q, _ = np.linalg.qr(rng.standard_normal((N, D)))
    norms = np.array([2.0 ** (-k / 2) for k in range(D)]) * 8       # bf16-exact scales
    x = q * norms[None, :]
    # bf16 rounding of x perturbs the columns: compare with tolerance of that rounding
    b, s = SV.basis(x, np.ones(N), 4)
    np.testing.assert_allclose(s, norms, rtol=2e-2)
    for i in range(4):
        assert abs(abs(b[i, i]) - 1) < 1e-2


def test_unit_weights_reduce_to_the_plain_svd_of_x():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 12)).astype(np.float32)
    xb = SV.weighted_rows(x, np.ones(40))          # bf16(x)
    b, s = SV.basis(x, np.ones(40), 12)
    u, s2, vt = np.linalg.svd(xb)
    np.testing.assert_allclose(s[:12], s2, rtol=1e-12)
    np.testing.assert_allclose(np.abs(b @ vt.T), np.eye(12), atol=1e-9)


def test_integer_weight_equals_repeating_the_sample():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 6)).astype(np.float32)
    w = np.ones(10)
    w[3] = 4.0                                      # sqrt(4) = 2: exact in bf16 scaling
    x_rep = np.concatenate([x, np.repeat(x[3:4], 3, axis=0)], axis=0)
    np.testing.assert_allclose(SV.gram(x, w), SV.gram(x_rep, np.ones(13)), rtol=1e-12, atol=1e-12)


def test_scaling_weights():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((30, 8))
    w = rng.uniform(0.1, 2.0, 30)
    b1, s1 = SV.basis(x, w, 5)
    b2, s2 = SV.basis(x, w * 4.0, 5)                # sqrt(4) = 2, a power of two: exact
    np.testing.assert_allclose(s2, 2 * s1, rtol=1e-12)
    np.testing.assert_allclose(b2, b1, atol=1e-9)


def test_rank_one_data_gives_its_direction():
    rng = np.random.default_rng(4)
    v = np.zeros(10)
    v[[1, 4, 7]] = [0.5, -0.25, 1.0]
    x = rng.standard_normal(25)[:, None] * v[None, :]
    b, s = SV.basis(x, rng.uniform(0.5, 1.5, 25), 1)
    np.testing.assert_allclose(np.abs(b[0]), np.abs(v) / np.linalg.norm(v), atol=1e-2)
    assert s[1] < 1e-2 * s[0]


@pytest.mark.parametrize("seed", [5, 6])
def test_beats_random_bases_on_the_weighted_error(seed):
    """Eckart-Young on the weighted rows: no rank-6 orthonormal basis reconstructs them better."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((80, 16)) * np.linspace(3, 0.2, 16)).astype(np.float32)
    w = rng.uniform(0.0, 3.0, 80)
    y = SV.weighted_rows(x, w)
    b, _ = SV.basis(x, w, 6)
    err = lambda bb: float(np.sum((y - y @ bb.T @ bb) ** 2))
    e = err(b)
    for _ in range(20):
        q, _ = np.linalg.qr(rng.standard_normal((16, 6)))
        assert err(q.T) >= e * (1 - 1e-12)
    # and a small rotation of the basis inside and outside its span does not help either
    pert, _ = np.linalg.qr((b + 1e-3 * rng.standard_normal(b.shape)).T)
    assert err(pert.T) >= e * (1 - 1e-12)


def test_zero_weight_samples_have_no_influence():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20, 8))
    w = rng.uniform(0.5, 1.5, 20)
    w2 = w.copy()
    w2[[2, 9]] = 0.0
    x2 = x.copy()
    x2[[2, 9]] = 1e3
    keep = np.ones(20, bool)
    keep[[2, 9]] = False
    np.testing.assert_allclose(SV.gram(x2, w2), SV.gram(x[keep], w[keep]), rtol=1e-12, atol=1e-12)
