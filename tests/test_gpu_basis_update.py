"""GPU parity of lowrank_basis_update (block-incremental basis update, iS-KV) against the oracle.

Two references:
  * the exact SVD (float64) of the very rows the library factorises, M~ = [bf16(sigma_i B_i) ; Y]:
    spectrum within 1e-5 sigma_max^2 (as the weighted-SVD tests), the top-r' projector within 1e-3,
    and well-separated rows one by one (sign convention included);
  * the oracle's incremental update (Brand's steps, float64) on the unrounded inputs: singular
    values within ||M~ - M||_2 (Weyl) and the projector within the Wedin bound, since M~ differs
    from M by the bf16 rounding of the weighted basis rows.
W = B' B^T is checked against the product of the call's own B' and B (float32 accumulation bound,
then the output rounding) and against the oracle's W row by row. A composition test runs update ->
coordinate sync (lowrank_kv_rebase with that W) -> decode against the oracle's composition.
"""
import dataclasses

import numpy as np
import pytest
import torch

import rank_kv_cache_lowrank_amd as lr
import synth
from oracle import append as OAP
from oracle import attention as OA
from oracle import basis_update as BU
from oracle import sensvd as SV

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(r, n, D=512, decay=0.93, y_scale=1.0, seed=0, dtype="f32"):
    cfg = synth.CONFIGS[4]
    B64 = synth.gen_basis(cfg.replace(cfg_id=70 + seed), "k", 0, r)          # orthonormal rows, float64
    Bst = synth.to_storage(B64, "f32" if dtype == "f32" else "bf16")
    sigma = (10.0 * decay ** np.arange(r)).astype(np.float32)
    rng = np.random.default_rng(100 + seed)
    Y = synth.to_storage(rng.standard_normal((n, D)) * y_scale, "bf16")
    return Bst, sigma, Y


def _run(Bst, sigma, Y, r_new, sweeps=0):
    r, D = Bst.shape
    n = 0 if Y is None else Y.shape[0]
    ws = torch.empty(lr.lowrank_basis_update_workspace_size(r, n, D), dtype=torch.uint8, device=DEV)
    bn = torch.full((r_new, D), float("nan"), dtype=Bst.dtype, device=DEV)
    sn = torch.full((r_new,), float("nan"), dtype=torch.float32, device=DEV)
    ldw = (r + 7) // 8 * 8
    w = torch.full((r_new, ldw), float("nan"), dtype=Bst.dtype, device=DEV)
    lr.lowrank_basis_update(Bst.to(DEV), torch.from_numpy(sigma).to(DEV), None if Y is None else Y.to(DEV), r_new,
                            bn, sn, w, ws, sweeps)
    torch.cuda.synchronize()
    return bn.double().cpu().numpy(), sn.double().cpu().numpy(), w.double().cpu().numpy()


def _staged_rows(Bst, sigma, Y):
    """The rows the library factorises: bf16(f32(sigma_i) * B_i) (one rounding), then Y."""
    top = OAP.bf16_rne((sigma[:, None].astype(np.float32) * Bst.float().numpy()).astype(np.float32))
    rows = [top.astype(np.float64)]
    if Y is not None:
        rows.append(Y.double().numpy())
    return np.concatenate(rows, axis=0)


def _projector(rows):
    return rows.T @ rows


def _residual(M, rows):
    """||M - M P||_F^2 with P the orthogonal projector onto the row space of `rows`."""
    Q = np.linalg.qr(rows.T)[0]
    R = M - (M @ Q) @ Q.T
    return float(np.sum(R * R))


@pytest.mark.parametrize("r,n,r_new,dtype", [(64, 32, 80, "f32"), (256, 128, 256, "f32"), (256, 128, 256, "bf16"),
                                             (100, 7, 64, "f32")])
def test_basis_update_matches_the_svd_and_the_oracle(r, n, r_new, dtype):
    Bst, sigma, Y = _inputs(r, n, dtype=dtype, seed=r + n, y_scale=0.2)
    bn, sn, w = _run(Bst, sigma, Y, r_new)
    D = Bst.shape[1]
    ldw = (r + 7) // 8 * 8
    assert np.all(np.isfinite(bn)) and np.all(np.isfinite(sn)) and np.all(np.isfinite(w))
    out_tol = 1e-3 if dtype == "f32" else 1e-2            # bf16 output rows carry 2^-9 rounding
    # (1) the exact SVD of the staged rows: spectrum, Eckart-Young optimality, separated rows
    Mt = _staged_rows(Bst, sigma, Y)
    _, s_t, vt_t = np.linalg.svd(Mt, full_matrices=False)
    smax2 = s_t[0] ** 2
    s2_err = np.max(np.abs(sn ** 2 - s_t[:r_new] ** 2)) / smax2
    assert s2_err <= 1e-5, s2_err
    if dtype == "f32":
        np.testing.assert_allclose(bn @ bn.T, np.eye(r_new), atol=1e-5)
    opt = float(np.sum(s_t[r_new:] ** 2))
    excess = (_residual(Mt, bn) - opt) / smax2
    print(f"r={r} n={n} r'={r_new} {dtype}: sigma^2 err {s2_err:.2e}, Eckart-Young excess {excess:.2e}", flush=True)
    assert excess <= (1e-5 if dtype == "f32" else 1e-4) * r_new
    s_pad = np.r_[s_t, 0.0]
    gaps = np.minimum(np.r_[np.inf, s_t[:r_new - 1] - s_t[1:r_new]], s_t[:r_new] - s_pad[1:r_new + 1])
    sep = np.nonzero(gaps > 0.02 * s_t[0])[0]
    assert sep.size > 0
    for k in sep[:8]:
        ref = SV._fix_signs(vt_t[k:k + 1])[0]
        assert np.max(np.abs(bn[k] - ref)) <= out_tol, (k, np.max(np.abs(bn[k] - ref)))
    # (2) the oracle's incremental update on the unrounded inputs, within the perturbation bounds
    B64 = Bst.double().numpy()
    b_ref, s_ref = BU.incremental_update(sigma.astype(np.float64), B64, Y.double().numpy(), r_new)
    M = np.concatenate([np.diag(sigma.astype(np.float64)) @ B64, Y.double().numpy()], axis=0)
    e2 = np.linalg.norm(Mt - M, 2)
    assert np.all(np.abs(sn - s_ref) <= e2 + 1e-5 * s_t[0])              # Weyl
    for k in sep[:8]:                                                     # Wedin, per separated row
        assert np.max(np.abs(bn[k] - b_ref[k])) <= 2 * e2 / gaps[k] + out_tol
    # (3) W = B' B^T: the call's own factors (float32 sum, then the output rounding) ...
    w_own = bn @ B64.T
    bound = D * 2.0 ** -24 * (np.abs(bn) @ np.abs(B64).T) + 1e-30
    if dtype == "bf16":
        # W is formed from the float32 B' before its storage rounding (2^-9 per element), then
        # rounded itself
        bound += 2.0 ** -9 * (np.abs(bn) @ np.abs(B64).T) + 2.0 ** -8 * np.abs(w_own)
    assert np.all(np.abs(w[:, :r] - w_own) <= bound)
    assert np.all(w[:, r:ldw] == 0)
    # ... and the oracle's, row by row on the separated rows
    w_ref = BU.sync_weights(B64, b_ref)
    for k in sep[:8]:
        assert np.max(np.abs(w[k, :r] - w_ref[k])) <= 2 * e2 / gaps[k] + out_tol


def test_no_new_rows_truncates_to_the_leading_rows():
    """No block (n = 0) and a basis of unit rows e_pi(i) with bf16-exact sigma: the staged rows are
    exactly diag(sigma) B, so B' is exactly the first r' rows of B, sigma' = sigma[:r'] and
    W = [I 0]."""
    r, r_new, D = 96, 40, 512
    rng = np.random.default_rng(3)
    B = np.zeros((r, D), np.float32)
    B[np.arange(r), rng.permutation(D)[:r]] = 1.0
    sigma = OAP.bf16_rne((10.0 * 0.93 ** np.arange(r)).astype(np.float32))
    for dtype in ("f32", "bf16"):
        Bst = synth.to_storage(B, dtype)
        bn, sn, w = _run(Bst, sigma, None, r_new)
        np.testing.assert_allclose(sn, sigma[:r_new], rtol=1e-6)
        np.testing.assert_allclose(bn, B[:r_new], atol=1e-6)
        np.testing.assert_allclose(w[:, :r], np.eye(r_new, r), atol=1e-6)


def test_rows_inside_the_span_keep_the_span():
    Bst, sigma, _ = _inputs(64, 0, seed=4, decay=0.97)
    rng = np.random.default_rng(4)
    B64 = Bst.double().numpy()
    Y = synth.to_storage(rng.standard_normal((16, 64)) @ B64, "bf16")
    bn, _, _ = _run(Bst, sigma, Y, 64)
    # Y's bf16 rounding moves it off span(B) by ~2^-9 of its size
    assert np.linalg.norm(_projector(bn) - _projector(B64), 2) <= 1e-2


def test_update_then_sync_then_decode_matches_the_oracle_composition():
    """float32 latents. A history whose basis rows are its principal axes (z = U diag(sigma) with
    orthonormal U, so X = z B is held exactly as U diag(sigma) B) takes a block of new rows drawn like
    its own tokens; fold it (r' = r + n, nothing truncated), sync every stored row with the call's W
    (lowrank_kv_rebase), decode with the new basis. References: the same composition with the call's
    own B' and W (checks the sync and the decode over them), and the oracle's update (Brand, float64,
    unrounded). Reading the stale coordinates in the new basis (no sync) is far off: the drift the
    pages describe."""
    cfg = synth.CONFIGS[0].replace(batch=2, seq_len=300, rank_k=96, rank_v=96)
    li0 = synth.make_layer(cfg, q_scale=4.0)
    r, n, D = 96, 24, 512
    r_new = r + n
    B_len = int(li0.lat_len.sum())
    rng = np.random.default_rng(12)

    def history(which):
        U = np.linalg.qr(rng.standard_normal((B_len, r)))[0]
        sig = np.sqrt(B_len / np.arange(1, r + 1))                 # the latents' own energy profile
        z = (U * sig[None, :]).astype(np.float32)
        return z, sig.astype(np.float32)

    zk_all, sig_k = history("k")
    zv_all, sig_v = history("v")
    zk = torch.from_numpy(synth.padded_rows([zk_all[:300], zk_all[300:]], li0.t_cap, li0.ld_k))
    zv = torch.from_numpy(synth.padded_rows([zv_all[:300], zv_all[300:]], li0.t_cap, li0.ld_v))
    li = dataclasses.replace(li0, zk=zk, zv=zv)
    # new rows: tokens like the history's (coordinates ~ a history row) plus a component outside span(B)
    Bk64, Bv64 = li.bk.double().numpy(), li.bv.double().numpy()
    Yk = synth.to_storage(zk_all[rng.integers(0, B_len, n)] @ Bk64 + 0.3 * rng.standard_normal((n, D)), "bf16")
    Yv = synth.to_storage(zv_all[rng.integers(0, B_len, n)] @ Bv64 + 0.3 * rng.standard_normal((n, D)), "bf16")
    bk_new, _, wk = _run(li.bk, sig_k, Yk, r_new)
    bv_new, _, wv = _run(li.bv, sig_v, Yv, r_new)
    # device sync of the stored rows
    model = lr.Model(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, [r], [r], cfg.sm_scale, 0, "f32")
    lat = torch.from_numpy(li.lat_len).to(DEV)
    src = lr.Cache(li.zk.to(DEV), li.zv.to(DEV), None, None, lat, li.t_cap, li.ld_k, li.ld_v)
    ld2 = synth.latent_ld(r_new)
    dk = torch.full((cfg.batch, li.t_cap, ld2), float("nan"), device=DEV)
    dv = torch.full((cfg.batch, li.t_cap, ld2), float("nan"), device=DEV)
    dst = lr.Cache(dk, dv, None, None, None, li.t_cap, ld2, ld2)
    wk_t = torch.from_numpy(wk.astype(np.float32)).to(DEV).contiguous()
    wv_t = torch.from_numpy(wv.astype(np.float32)).to(DEV).contiguous()
    lr.lowrank_kv_rebase(model, 0, src, dst, int(li.lat_len.max()), r_new, r_new, wk_t, wv_t)
    # decode with the new basis over the synced rows
    model2 = lr.Model(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, [r_new], [r_new], cfg.sm_scale, 0, "f32")
    c2 = lr.Cache(dk, dv, torch.from_numpy(bk_new.astype(np.float32)).to(DEV),
                  torch.from_numpy(bv_new.astype(np.float32)).to(DEV), lat, li.t_cap, ld2, ld2)
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, device=DEV)
    ws = lr.workspace(model2, 0, cfg.batch, int(li.lat_len.max()))
    lr.lowrank_attn_decode(model2, 0, c2, li.q.to(DEV), out, int(li.lat_len.max()), ws)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    q = li.q.double().numpy()
    zks = [li.zk[b, :li.lat_len[b], :r].double().numpy() for b in range(cfg.batch)]
    zvs = [li.zv[b, :li.lat_len[b], :r].double().numpy() for b in range(cfg.batch)]

    def attend(zk_, zv_, bk_, bv_, rk_, rv_):
        return OA.decode_latent(q, zk_, zv_, bk_, bv_, li.lat_len, rk_, rv_, cfg.n_kv_heads, cfg.sm_scale)

    def rel(a, b):
        return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))

    mech = attend([z @ wk[:, :r].T for z in zks], [z @ wv[:, :r].T for z in zvs], bk_new, bv_new, r_new, r_new)
    ref_k, _ = BU.incremental_update(sig_k.astype(np.float64), Bk64, Yk.double().numpy(), r_new)
    ref_v, _ = BU.incremental_update(sig_v.astype(np.float64), Bv64, Yv.double().numpy(), r_new)
    ref = attend([z @ BU.sync_weights(Bk64, ref_k).T for z in zks], [z @ BU.sync_weights(Bv64, ref_v).T for z in zvs],
                 ref_k, ref_v, r_new, r_new)
    orig = attend(zks, zvs, Bk64, Bv64, r, r)
    stale = attend([np.pad(z, ((0, 0), (0, n))) for z in zks], [np.pad(z, ((0, 0), (0, n))) for z in zvs],
                   ref_k, ref_v, r_new, r_new)
    err_mech, err, drift_gpu, drift_stale = rel(got, mech), rel(got, ref), rel(got, orig), rel(stale, orig)
    print(f"update->sync->decode: vs own factors {err_mech:.3e}, vs oracle update {err:.3e}; drift from the "
          f"original history: synced {drift_gpu:.3e}, stale {drift_stale:.3e}", flush=True)
    assert err_mech <= 5e-3
    assert err <= 1e-2          # B' from the bf16-staged rows vs the exact update: 2^-9 row perturbations
    assert drift_gpu <= 1e-2    # nothing was truncated: the synced history is the original one
    assert drift_stale > 0.2
