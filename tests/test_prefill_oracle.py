"""Pins of the chunked-prefill oracle (oracle/prefill.py): closed forms, a library routine,
the decode oracle, invariants and brute force."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import prefill as P


def rand_case(seed, B=2, C=5, Hq=8, Hkv=2, d=8, rk=6, rv=5, L=(7, 0), window=0, wl=None):
    rng = np.random.default_rng(seed)
    D = Hkv * d
    T = max(L) + 1
    c = dict(q=rng.standard_normal((B, C, Hq, d)), zk=rng.standard_normal((B, T, rk)),
             zv=rng.standard_normal((B, T, rv)), bk=rng.standard_normal((rk, D)) / math.sqrt(rk),
             bv=rng.standard_normal((rv, D)) / math.sqrt(rv), lat_len=list(L), rank_k=rk, rank_v=rv,
             n_kv_heads=Hkv, sm_scale=1 / math.sqrt(d), k_new=rng.standard_normal((B, C, D)),
             v_new=rng.standard_normal((B, C, D)))
    if window:
        c.update(kwin=rng.standard_normal((B, window, D)), vwin=rng.standard_normal((B, window, D)),
                 win_len=list(wl), window=window)
    return c


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("window,wl", [(0, None), (4, [4, 2]), (4, [0, 3])])
def test_p1_equals_p2(window, wl):
    c = rand_case(1, window=window, wl=wl)
    assert rel(P.prefill_latent(**c), P.prefill_reconstruct(**c)) < 1e-12


def test_identity_bases_equal_masked_sdpa():
    """Full rank with identity bases: dense GQA attention of the chunk's queries, aligned with
    the end of the key sequence (history, then the causal chunk)."""
    rng = np.random.default_rng(3)
    B, C, Hq, Hkv, d, T = 2, 6, 28, 4, 128, 40
    D = Hkv * d
    q = rng.standard_normal((B, C, Hq, d))
    Z = rng.standard_normal((B, T, D))
    Zv = rng.standard_normal((B, T, D))
    kn = rng.standard_normal((B, C, D))
    vn = rng.standard_normal((B, C, D))
    eye = np.eye(D)
    lens = [T, 13]
    kw = dict(q=q, zk=Z, zv=Zv, bk=eye, bv=eye, lat_len=lens, rank_k=D, rank_v=D, n_kv_heads=Hkv,
              sm_scale=1 / math.sqrt(d), k_new=kn, v_new=vn)
    for fn in (P.prefill_reconstruct, P.prefill_latent):
        out = fn(**kw)
        for b, L in enumerate(lens):
            K = np.concatenate([Z[b, :L], kn[b]], 0)
            V = np.concatenate([Zv[b, :L], vn[b]], 0)
            n = L + C
            mask = np.zeros((C, n), bool)
            for cc in range(C):
                mask[cc, :L + cc + 1] = True
            grp = Hq // Hkv
            Kh = torch.from_numpy(K.reshape(n, Hkv, d).transpose(1, 0, 2).repeat(grp, 0).copy())
            Vh = torch.from_numpy(V.reshape(n, Hkv, d).transpose(1, 0, 2).repeat(grp, 0).copy())
            qh = torch.from_numpy(q[b].transpose(1, 0, 2).copy())              # [Hq, C, d]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh, Kh, Vh, attn_mask=torch.from_numpy(mask), scale=1 / math.sqrt(d))
            assert rel(out[b], ref.numpy().transpose(1, 0, 2)) < 1e-12


@pytest.mark.parametrize("window,wl", [(0, None), (6, [3, 0])])
def test_one_token_chunk_equals_decode_with_the_token_in_the_window(window, wl):
    c = rand_case(4, C=1, window=window, wl=wl)
    out = P.prefill_reconstruct(**c)
    # decode oracle: the chunk token becomes the newest exact window token
    B, _, Hq, d = c["q"].shape
    D = c["k_new"].shape[-1]
    W2 = (window or 0) + 1
    kw2 = np.zeros((B, W2, D))
    vw2 = np.zeros((B, W2, D))
    wl2 = []
    for b in range(B):
        L = c["lat_len"][b]
        n_old = wl[b] if window else 0
        rows_k = [c["kwin"][b][(L + i) % window] for i in range(n_old)] if window else []
        rows_v = [c["vwin"][b][(L + i) % window] for i in range(n_old)] if window else []
        rows_k.append(c["k_new"][b, 0])
        rows_v.append(c["v_new"][b, 0])
        for i, (rk_, rv_) in enumerate(zip(rows_k, rows_v)):
            kw2[b, (L + i) % W2] = rk_
            vw2[b, (L + i) % W2] = rv_
        wl2.append(len(rows_k))
    dec = A.decode_reconstruct(c["q"][:, 0], c["zk"], c["zv"], c["bk"], c["bv"], c["lat_len"], c["rank_k"],
                               c["rank_v"], c["n_kv_heads"], c["sm_scale"], kwin=kw2, vwin=vw2, win_len=wl2,
                               window=W2)
    assert rel(out[:, 0], dec) < 1e-12


def test_causality():
    c = rand_case(5, C=6)
    out = P.prefill_latent(**c)
    c2 = dict(c)
    c2["k_new"] = c["k_new"].copy()
    c2["v_new"] = c["v_new"].copy()
    c2["k_new"][:, 3:] += 10.0
    c2["v_new"][:, 3:] -= 7.0
    out2 = P.prefill_latent(**c2)
    np.testing.assert_array_equal(out[:, :3], out2[:, :3])
    assert rel(out[:, 3:], out2[:, 3:]) > 1e-3


def test_first_token_of_an_empty_cache_returns_its_value():
    c = rand_case(6, B=1, L=(0,))
    out = P.prefill_reconstruct(**c)
    Hq, d = c["q"].shape[2:]
    grp = Hq // c["n_kv_heads"]
    for j in range(Hq):
        g = j // grp
        np.testing.assert_allclose(out[0, 0, j], c["v_new"][0, 0, g * d:(g + 1) * d], atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_bruteforce(seed):
    c = rand_case(10 + seed, B=2, C=3, Hq=4, Hkv=2, d=3, rk=3, rv=2, L=(4, 1))
    ref = np.array(P.prefill_bruteforce(c["q"], c["zk"], c["zv"], c["bk"], c["bv"], c["lat_len"], c["rank_k"],
                                        c["rank_v"], c["n_kv_heads"], c["sm_scale"], c["k_new"], c["v_new"]))
    assert rel(P.prefill_reconstruct(**c), ref) < 1e-12
    assert rel(P.prefill_latent(**c), ref) < 1e-12


def test_a_slip_in_the_latent_steps_is_caught_by_the_dense_pin():
    """Plant a transposed value basis in a copy of P2 and check that P1 disagrees."""
    c = rand_case(7, rk=5, rv=5)
    bad = dict(c)
    bad["bv"] = c["bv"].copy()
    bad["bv"][:, :] = bad["bv"][::-1]          # wrong row order of Bv
    assert rel(P.prefill_latent(**bad), P.prefill_reconstruct(**c)) > 1e-3
