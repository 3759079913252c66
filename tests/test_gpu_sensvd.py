"""GPU parity of lowrank_sens_svd (sensitivity-weighted SVD basis) against the oracle: squared
singular values within 1e-6 of the largest, basis rows orthonormal to 1e-5, each row an eigenvector of the
oracle's Gram (residual 1e-4 of the top eigenvalue), and the top-r subspace equal to the oracle's
where the spectrum has a gap there."""
import numpy as np
import pytest
import torch

import synth
import rank_kv_cache_lowrank_amd as lr
from oracle import sensvd as SV

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(x, w, rank, basis_dtype=torch.float32, sweeps=0):
    n, dim = x.shape
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(DEV)
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV)
    basis = torch.full((rank, dim), float("nan"), dtype=basis_dtype, device=DEV)
    sigma = torch.empty(dim, dtype=torch.float32, device=DEV)
    ws = torch.empty(lr.lowrank_sens_svd_workspace_size(n, dim), dtype=torch.uint8, device=DEV)
    lr.lowrank_sens_svd(xd, wd, rank, basis, sigma, ws, sweeps=sweeps)
    torch.cuda.synchronize()
    return basis.float().cpu().numpy().astype(np.float64), sigma.cpu().numpy().astype(np.float64)


def check(x, w, rank, b, s, gap_at_rank=True, tol_sigma=1e-6):
    xb = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()   # stored rows
    b_ref, s_ref = SV.basis(xb, w, rank)
    G = SV.gram(xb, w)
    lam_max = max(float(s_ref[0]) ** 2, 1e-30)
    # eigenvalues are Rayleigh quotients on the float32 Gram: their error is that of the quadratic
    # form v^T G v, where the entries' independent roundings largely cancel (measured <= 1e-7
    # lambda_max up to 131072 samples). Bound: |sigma^2 - sigma_ref^2| <= 1e-6 lambda_max, so
    # zero singular values read <= 1e-3 sigma_max.
    assert np.max(np.abs(s * s - s_ref * s_ref)) <= tol_sigma * lam_max + 1e-30
    assert np.all(np.diff(s) <= 0)
    np.testing.assert_allclose(b @ b.T, np.eye(rank), atol=1e-5)
    lam = np.sum((b @ G) * b, axis=1)
    res = np.linalg.norm(b @ G - lam[:, None] * b, axis=1)
    assert np.max(res) <= 1e-4 * lam_max
    if gap_at_rank:
        P = b.T @ b
        P_ref = b_ref.T @ b_ref
        assert np.linalg.norm(P - P_ref, 2) < 1e-3


@pytest.mark.parametrize("n,dim,rank,decay", [(4096, 512, 358, 1.0), (1000, 256, 64, 0.8), (70, 128, 128, 1.5),
                                               (300, 64, 10, 0.5)])
def test_matches_oracle(n, dim, rank, decay):
    cfg = synth.CONFIGS[4]
    x, w = synth.gen_kv_samples(cfg, n, dim, decay)
    b, s = run(x, w, rank)
    check(x, w, rank, b, s, gap_at_rank=(rank < dim))


def test_gapped_spectrum_rows_match_one_by_one():
    """Well-separated singular values: each row equals the oracle's (same sign convention)."""
    rng = np.random.default_rng(3)
    dim, n = 64, 512
    q, _ = np.linalg.qr(rng.standard_normal((dim, dim)))
    sv = 2.0 ** (-np.arange(dim) / 4.0)
    x = (rng.standard_normal((n, dim)) * sv) @ q.T
    w = rng.uniform(0.5, 2.0, n)
    b, s = run(x, w, 16)
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    b_ref, s_ref = SV.basis(xb, w, 16)
    for k in range(16):
        assert abs(abs(float(b[k] @ b_ref[k])) - 1) < 1e-4
    np.testing.assert_allclose(b, b_ref, atol=2e-3)


def test_bf16_basis_output():
    x, w = synth.gen_kv_samples(synth.CONFIGS[4], 800, 128, 1.0)
    b32, s32 = run(x, w, 32)
    b16, s16 = run(x, w, 32, basis_dtype=torch.bfloat16)
    np.testing.assert_array_equal(s16, s32)
    np.testing.assert_array_equal(b16, torch.from_numpy(b32).to(torch.bfloat16).double().numpy())


def test_zero_weights_and_ragged_counts():
    x, w = synth.gen_kv_samples(synth.CONFIGS[4], 33, 64, 1.0)
    b, s = run(x, np.zeros_like(w), 8)
    assert np.all(s == 0)
    for n in (1, 31, 257):
        x, w = synth.gen_kv_samples(synth.CONFIGS[4], n, 64, 1.0)
        b, s = run(x, w, 8)
        check(x, w, 8, b, s, gap_at_rank=False)


def test_rank_one_data():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(128)
    x = rng.standard_normal(200)[:, None] * v[None, :]
    b, s = run(x, rng.uniform(0.5, 1.5, 200), 1)
    vb = torch.from_numpy(v.astype(np.float32)).float().numpy()
    assert abs(abs(float(b[0] @ vb)) / np.linalg.norm(vb) - 1) < 1e-3
    assert s[1] < 1e-2 * s[0]


def test_full_calibration_shape():
    """256 samples x 512 tokens of one KV matrix (131072 rows, dim 512), rank 358."""
    x, w = synth.gen_kv_samples(synth.CONFIGS[4], 131072, 512, 1.0)
    b, s = run(x, w, 358)
    check(x, w, 358, b, s)


@pytest.mark.parametrize("n_mat,n,dim,rank", [(3, 1000, 256, 64), (4, 4096, 512, 358)])
def test_batched_equals_single_calls(n_mat, n, dim, rank):
    """lowrank_sens_svd_batched: matrix m's basis and spectrum are bit-identical to a single call on
    its slices (the same kernels), and match the oracle."""
    xs, ws_ = [], []
    for m in range(n_mat):
        x, w = synth.gen_kv_samples(synth.CONFIGS[4], n, dim, 0.6 + 0.2 * m)
        xs.append(x)
        ws_.append(w)
    xd = torch.from_numpy(np.stack(xs).astype(np.float32)).to(torch.bfloat16).to(DEV)
    wd = torch.from_numpy(np.stack(ws_).astype(np.float32)).to(DEV)
    basis = torch.full((n_mat, rank, dim), float("nan"), dtype=torch.float32, device=DEV)
    sigma = torch.empty(n_mat, dim, dtype=torch.float32, device=DEV)
    ws = torch.empty(lr.lowrank_sens_svd_batched_workspace_size(n_mat, n, dim), dtype=torch.uint8, device=DEV)
    lr.lowrank_sens_svd_batched(xd, wd, rank, basis, sigma, ws)
    torch.cuda.synchronize()
    for m in range(n_mat):
        b1, s1 = run(xs[m], ws_[m], rank)
        np.testing.assert_array_equal(basis[m].cpu().numpy().astype(np.float64), b1)
        np.testing.assert_array_equal(sigma[m].cpu().numpy().astype(np.float64), s1)
        check(xs[m], ws_[m], rank, b1, s1, gap_at_rank=rank < dim)


def test_invalid_arguments():
    x = torch.zeros(16, 96, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(16, device=DEV)
    basis = torch.empty(8, 96, device=DEV)
    sigma = torch.empty(96, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(lr.LowRankError):
        lr.lowrank_sens_svd(x, w, 8, basis, sigma, ws)        # dim not a multiple of 64
    assert lr.lowrank_sens_svd_workspace_size(16, 96) == 0
