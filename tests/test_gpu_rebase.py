"""GPU parity of lowrank_kv_rebase (historical-coordinate sync) against the oracle.

Bit-exact where every new coordinate is exact in any summation order (signed power-of-two
permutation W); otherwise within half a bf16 ulp of the float64 result plus the float32
accumulation bound r * 2^-24 * sum |z_i w_ji|. Rows past lat_len and columns past the new rank
must keep their NaN sentinels.
"""
import numpy as np
import pytest
import torch

import synth
import rank_kv_cache_lowrank_amd as lr
from oracle import rebase as RB
from helpers import TOL, oracle_decode, rel_err, run_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")


def latents(rng, B, t_cap, r, ld, latent, lat_len):
    """Stored rows N(0,1)/sqrt(i) in [0, lat_len[b]); NaN in pad columns and rows past it."""
    z = np.full((B, t_cap, ld), np.nan, np.float32)
    for b in range(B):
        L = int(lat_len[b])
        z[b, :L, :r] = rng.standard_normal((L, r)).astype(np.float32) / np.sqrt(np.arange(1, r + 1))
    return synth.to_storage(z, latent).to(DEV)


def new_buffer(B, t_cap, ld, latent):
    dt = torch.float32 if latent == "f32" else torch.bfloat16
    return torch.full((B, t_cap, ld), NAN, dtype=dt, device=DEV)


def make(latent, B, t_cap, rk, rv, lat_len, seed=0):
    rng = np.random.default_rng(seed)
    ldk, ldv = synth.latent_ld(rk), synth.latent_ld(rv)
    zk = latents(rng, B, t_cap, rk, ldk, latent, lat_len)
    zv = latents(rng, B, t_cap, rv, ldv, latent, lat_len)
    lat = torch.from_numpy(np.asarray(lat_len, np.int32)).to(DEV)
    model = lr.Model(1, 28, 4, 128, [rk], [rv], 128 ** -0.5, 0, latent)
    return model, lr.Cache(zk, zv, None, None, lat, t_cap, ldk, ldv)


def random_w(rng, rn, r, scale=1.0):
    return rng.standard_normal((rn, r)) * (scale / np.sqrt(r))


def signed_pow2_perm(rng, rn, r):
    """Each new coordinate is +-2^k times one old coordinate (or 0): exact in any order."""
    w = np.zeros((rn, r))
    perm = rng.permutation(max(r, rn))
    for j in range(rn):
        if perm[j] < r:
            w[j, perm[j]] = rng.choice([-1.0, 1.0]) * 2.0 ** int(rng.integers(-3, 4))
    return w


def expect(z_old, w_stored, latent):
    """Oracle rows (float64 exact and stored form) from the stored inputs."""
    z64 = z_old.astype(np.float64)
    exact = RB.rebase_rows(z64, w_stored.astype(np.float64))
    return exact, RB.store(exact, latent)


def check_rows(got, z_old, w_stored, latent, exact_bits=False):
    if got.size == 0:
        return
    exact, stored = expect(z_old, w_stored, latent)
    if exact_bits:
        np.testing.assert_array_equal(got, stored)
        return
    r = z_old.shape[1]
    acc = r * 2.0 ** -24 * (np.abs(z_old.astype(np.float64)) @ np.abs(w_stored.astype(np.float64)).T)
    if latent == "bf16":
        mag = np.abs(exact) + acc
        half_ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 8), 0.0)
        bound = acc + half_ulp
    else:
        bound = acc + np.abs(exact) * 2.0 ** -24
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= bound * 1.0001 + 1e-30), f"max excess {np.max(err - bound)}"
    if latent == "bf16":
        # only values within the accumulation bound of a rounding boundary may differ
        assert np.mean(got == stored) > 0.97


def run(model, src, dst, max_len, rk_new, rv_new, wk, wv):
    lr.lowrank_kv_rebase(model, 0, src, dst, max_len, rk_new, rv_new, wk, wv)
    torch.cuda.synchronize()


def host(t):
    return t.float().cpu().numpy()


def check_all(latent, src_host, dst_t, lat_len, r_old, r_new, w_host, exact_bits=False):
    got = host(dst_t)
    B = got.shape[0]
    for b in range(B):
        L = int(lat_len[b])
        check_rows(got[b, :L, :r_new], src_host[b, :L, :r_old], w_host, latent, exact_bits)
        assert np.isnan(got[b, L:]).all(), "rebase wrote rows past lat_len"
        assert np.isnan(got[b, :L, r_new:]).all(), "rebase wrote columns past the new rank"


@pytest.mark.parametrize("rk,rv,rk2,rv2", [
    (358, 358, 358, 358), (256, 256, 256, 256), (512, 512, 512, 512), (1, 33, 33, 1),
    (100, 64, 512, 80), (512, 130, 7, 200), (32, 48, 40, 16), (200, 300, 144, 460), (256, 250, 512, 400)])
def test_bf16_general_update(rk, rv, rk2, rv2):
    lat_len = [0, 1, 31, 32, 33, 95, 300, 517]
    B, t_cap = len(lat_len), 520
    model, src = make("bf16", B, t_cap, rk, rv, lat_len, seed=rk * 7 + rv2)
    rng = np.random.default_rng(rk2 + 1000 * rv)
    wk = synth.w_storage(random_w(rng, rk2, rk), "bf16", fill=NAN).to(DEV)
    wv = synth.w_storage(random_w(rng, rv2, rv), "bf16", fill=NAN).to(DEV)
    dk = new_buffer(B, t_cap, synth.latent_ld(rk2), "bf16")
    dv = new_buffer(B, t_cap, synth.latent_ld(rv2), "bf16")
    dst = lr.Cache(dk, dv, None, None, None, t_cap, synth.latent_ld(rk2), synth.latent_ld(rv2))
    zk_h, zv_h = host(src.zk), host(src.zv)
    run(model, src, dst, max(lat_len), rk2, rv2, wk, wv)
    check_all("bf16", zk_h, dk, lat_len, rk, rk2, host(wk)[:, :rk])
    check_all("bf16", zv_h, dv, lat_len, rv, rv2, host(wv)[:, :rv])
    # the source is untouched out of place
    np.testing.assert_array_equal(host(src.zk)[~np.isnan(zk_h)], zk_h[~np.isnan(zk_h)])


@pytest.mark.parametrize("rk,rk2", [(358, 358), (512, 480), (64, 512), (256, 255)])
def test_bf16_signed_permutation_is_bit_exact(rk, rk2):
    lat_len = [70, 1, 64, 129]
    B, t_cap = len(lat_len), 130
    model, src = make("bf16", B, t_cap, rk, rk, lat_len, seed=3)
    rng = np.random.default_rng(rk2)
    wk = synth.w_storage(signed_pow2_perm(rng, rk2, rk), "bf16", fill=NAN).to(DEV)
    wv = synth.w_storage(signed_pow2_perm(rng, rk2, rk), "bf16", fill=NAN).to(DEV)
    ld2 = synth.latent_ld(rk2)
    dk, dv = new_buffer(B, t_cap, ld2, "bf16"), new_buffer(B, t_cap, ld2, "bf16")
    dst = lr.Cache(dk, dv, None, None, None, t_cap, ld2, ld2)
    zk_h, zv_h = host(src.zk), host(src.zv)
    run(model, src, dst, max(lat_len), rk2, rk2, wk, wv)
    check_all("bf16", zk_h, dk, lat_len, rk, rk2, host(wk)[:, :rk], exact_bits=True)
    check_all("bf16", zv_h, dv, lat_len, rk, rk2, host(wv)[:, :rk], exact_bits=True)


@pytest.mark.parametrize("latent,rk,rv,rk2,rv2", [
    ("bf16", 358, 358, 192, 160), ("bf16", 358, 300, 352, 300), ("bf16", 40, 96, 32, 88),
    ("bf16", 512, 512, 128, 8),
    ("f32", 128, 128, 128, 128), ("f32", 48, 20, 40, 9)])
def test_in_place(latent, rk, rv, rk2, rv2):
    lat_len = [33, 0, 200, 17]
    B, t_cap = len(lat_len), 210
    model, src = make(latent, B, t_cap, rk, rv, lat_len, seed=11)
    rng = np.random.default_rng(5)
    wk = synth.w_storage(random_w(rng, rk2, rk), latent, fill=NAN).to(DEV)
    wv = synth.w_storage(random_w(rng, rv2, rv), latent, fill=NAN).to(DEV)
    zk_h, zv_h = host(src.zk), host(src.zv)
    run(model, src, src, max(lat_len), rk2, rv2, wk, wv)
    gk, gv = host(src.zk), host(src.zv)
    for b, L in enumerate(lat_len):
        check_rows(gk[b, :L, :rk2], zk_h[b, :L, :rk], host(wk)[:, :rk], latent)
        check_rows(gv[b, :L, :rv2], zv_h[b, :L, :rv], host(wv)[:, :rv], latent)
        # the old coordinates past the new rank and the rows past lat_len stay as they were
        np.testing.assert_array_equal(np.nan_to_num(gk[b, :L, rk2:], nan=7.0), np.nan_to_num(zk_h[b, :L, rk2:], nan=7.0))
        assert np.isnan(gk[b, L:]).all() and np.isnan(gv[b, L:]).all()


def test_in_place_too_wide_is_rejected():
    model, src = make("bf16", 1, 16, 512, 512, [16])
    w = synth.w_storage(np.zeros((512, 512)), "bf16").to(DEV)
    with pytest.raises(lr.LowRankError) as e:
        lr.lowrank_kv_rebase(model, 0, src, src, 16, 512, 512, w, w)
    assert e.value.code == lr.LR_EUNSUPPORTED


@pytest.mark.parametrize("rk,rv,rk2,rv2", [(128, 128, 128, 128), (48, 20, 64, 9), (1, 512, 512, 1)])
def test_f32_general_update(rk, rv, rk2, rv2):
    lat_len = [5, 64, 0]
    B, t_cap = len(lat_len), 70
    model, src = make("f32", B, t_cap, rk, rv, lat_len, seed=2)
    rng = np.random.default_rng(8)
    wk = synth.w_storage(random_w(rng, rk2, rk), "f32", fill=NAN).to(DEV)
    wv = synth.w_storage(random_w(rng, rv2, rv), "f32", fill=NAN).to(DEV)
    dk = new_buffer(B, t_cap, synth.latent_ld(rk2), "f32")
    dv = new_buffer(B, t_cap, synth.latent_ld(rv2), "f32")
    dst = lr.Cache(dk, dv, None, None, None, t_cap, synth.latent_ld(rk2), synth.latent_ld(rv2))
    zk_h, zv_h = host(src.zk), host(src.zv)
    run(model, src, dst, max(lat_len), rk2, rv2, wk, wv)
    check_all("f32", zk_h, dk, lat_len, rk, rk2, host(wk)[:, :rk])
    check_all("f32", zv_h, dv, lat_len, rv, rv2, host(wv)[:, :rv])


def test_lat_len_beyond_max_len_is_clamped():
    """Rows are bounded by max_lat_len even when a lat_len entry exceeds it."""
    lat_len = [40, 100]
    B, t_cap = 2, 100
    model, src = make("bf16", B, t_cap, 64, 64, lat_len, seed=4)
    w = synth.w_storage(np.eye(64), "bf16").to(DEV)
    dk, dv = new_buffer(B, t_cap, 64, "bf16"), new_buffer(B, t_cap, 64, "bf16")
    dst = lr.Cache(dk, dv, None, None, None, t_cap, 64, 64)
    run(model, src, dst, 50, 64, 64, w, w)
    got = host(dk)
    np.testing.assert_array_equal(got[0, :40], host(src.zk)[0, :40])
    np.testing.assert_array_equal(got[1, :50], host(src.zk)[1, :50])
    assert np.isnan(got[1, 50:]).all() and np.isnan(got[0, 40:]).all()


def test_full_size_sampled_rows():
    """16 sequences x 4096 rows at rank 358 (the r358 workload), 358 -> 358, sampled rows."""
    cfg = synth.CONFIGS[1]
    B, T, r = cfg.batch, cfg.seq_len, cfg.rank_k
    li = synth.make_layer(cfg)
    b_new_k = synth.gen_basis_update(cfg, "k", 0, li.bk.double().numpy(), r)
    b_new_v = synth.gen_basis_update(cfg, "v", 0, li.bv.double().numpy(), r)
    wk = synth.w_storage(synth.sync_projection(li.bk.double().numpy(), b_new_k), "bf16").to(DEV)
    wv = synth.w_storage(synth.sync_projection(li.bv.double().numpy(), b_new_v), "bf16").to(DEV)
    model = lr.Model(1, 28, 4, 128, [r], [r], cfg.sm_scale, 0, "bf16")
    lat = torch.from_numpy(li.lat_len).to(DEV)
    src = lr.Cache(li.zk.to(DEV), li.zv.to(DEV), None, None, lat, T, li.ld_k, li.ld_v)
    dk, dv = new_buffer(B, T, li.ld_k, "bf16"), new_buffer(B, T, li.ld_v, "bf16")
    dst = lr.Cache(dk, dv, None, None, None, T, li.ld_k, li.ld_v)
    run(model, src, dst, T, r, r, wk, wv)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, T, size=64)
    for b in range(B):
        sel = np.concatenate([rows, [0, T - 1]])
        for z, d, w in ((li.zk, dk, wk), (li.zv, dv, wv)):
            zo = z[b, sel, :r].float().numpy()
            got = d[b, torch.from_numpy(sel).to(DEV), :r].float().cpu().numpy()
            check_rows(got, zo, host(w)[:, :r], "bf16")


@pytest.mark.parametrize("r_new", [358, 300])
def test_decode_after_rebase_matches_oracle(r_new):
    """Rebase to B' then decode with B': the GPU composition equals the oracle's."""
    cfg = synth.CONFIGS[1].replace(batch=3, seq_len=300)
    li = synth.make_layer(cfg)
    r = li.rank_k
    bk64, bv64 = li.bk.double().numpy(), li.bv.double().numpy()
    b_new_k = synth.gen_basis_update(cfg, "k", 0, bk64, r_new)
    b_new_v = synth.gen_basis_update(cfg, "v", 0, bv64, r_new)
    wk = synth.w_storage(synth.sync_projection(bk64, b_new_k), "bf16").to(DEV)
    wv = synth.w_storage(synth.sync_projection(bv64, b_new_v), "bf16").to(DEV)
    model = lr.Model(1, 28, 4, 128, [r], [r], cfg.sm_scale, 0, "bf16")
    lat = torch.from_numpy(li.lat_len).to(DEV)
    src = lr.Cache(li.zk.to(DEV), li.zv.to(DEV), None, None, lat, li.t_cap, li.ld_k, li.ld_v)
    ld2 = synth.latent_ld(r_new)
    dk, dv = new_buffer(cfg.batch, li.t_cap, ld2, "bf16"), new_buffer(cfg.batch, li.t_cap, ld2, "bf16")
    dst = lr.Cache(dk, dv, None, None, None, li.t_cap, ld2, ld2)
    run(model, src, dst, int(li.lat_len.max()), r_new, r_new, wk, wv)

    # decode with the new basis on the GPU-rebased cache
    bk_new = synth.to_storage(b_new_k, "bf16")
    bv_new = synth.to_storage(b_new_v, "bf16")
    model2 = lr.Model(1, 28, 4, 128, [r_new], [r_new], cfg.sm_scale, 0, "bf16")
    cache2 = lr.Cache(torch.nan_to_num(dk), torch.nan_to_num(dv), bk_new.to(DEV), bv_new.to(DEV), lat,
                      li.t_cap, ld2, ld2)
    out = run_decode(model2, cache2, li.q.to(DEV), int(li.lat_len.max()))

    # the oracle composition: oracle-rebased stored rows, decoded with the new basis
    zk2 = np.zeros((cfg.batch, li.t_cap, ld2), np.float32)
    zv2 = np.zeros_like(zk2)
    for b in range(cfg.batch):
        L = int(li.lat_len[b])
        zk2[b, :L, :r_new] = RB.store(RB.rebase_rows(li.zk[b, :L, :r].float().numpy(), host(wk)[:, :r]), "bf16")
        zv2[b, :L, :r_new] = RB.store(RB.rebase_rows(li.zv[b, :L, :r].float().numpy(), host(wv)[:, :r]), "bf16")
    li2 = synth.LayerInputs(cfg=cfg, layer=0, rank_k=r_new, rank_v=r_new, ld_k=ld2, ld_v=ld2, t_cap=li.t_cap,
                            q=li.q, zk=synth.to_storage(zk2, "bf16"), zv=synth.to_storage(zv2, "bf16"),
                            bk=bk_new, bv=bv_new, lat_len=li.lat_len, win_len=li.win_len, kwin=None, vwin=None)
    ref = oracle_decode(li2)
    assert rel_err(out.numpy(), ref) < TOL["bf16"]
