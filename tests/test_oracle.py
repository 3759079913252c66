"""Pins of the decode-attention oracle (D1, D2, D3) against facts fixed outside it.

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, the
wrong KV group, a transposed basis, a lost window term, a softmax over the wrong
axis) fails at least one of them; ``test_pins_catch_planted_mistakes`` plants
such slips in copies of the oracle and checks that.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import synth
from oracle import attention as A


def rand_case(seed, B=2, Hq=28, Hkv=4, d=128, L=(37, 64), rk=40, rv=24, window=0, wl=None):
    rng = np.random.default_rng(seed)
    D = Hkv * d
    T = max(L)
    q = rng.standard_normal((B, Hq, d)) * 0.5
    zk = rng.standard_normal((B, T, rk))
    zv = rng.standard_normal((B, T, rv))
    bk = rng.standard_normal((rk, D)) / math.sqrt(D)
    bv = rng.standard_normal((rv, D)) / math.sqrt(D)
    kw = vw = None
    if window:
        kw = rng.standard_normal((B, window, D))
        vw = rng.standard_normal((B, window, D))
    return dict(q=q, zk=zk, zv=zv, bk=bk, bv=bv, lat_len=list(L), rank_k=rk, rank_v=rv,
                n_kv_heads=Hkv, sm_scale=1 / math.sqrt(d), kwin=kw, vwin=vw,
                win_len=wl if wl is not None else [window] * B, window=window)


def sdpa_dense(q, K, V, n_kv_heads, sm_scale):
    """Dense GQA attention through torch's library routine (CPU, float64).
    q [Hq, d]; K, V [T, Hkv*d] -> [Hq, d]."""
    Hq, d = q.shape
    T = K.shape[0]
    grp = Hq // n_kv_heads
    Kh = torch.from_numpy(K).reshape(T, n_kv_heads, d).permute(1, 0, 2)
    Vh = torch.from_numpy(V).reshape(T, n_kv_heads, d).permute(1, 0, 2)
    Kh = Kh.repeat_interleave(grp, dim=0).contiguous()   # HF repeat_kv: head j uses KV head j // grp
    Vh = Vh.repeat_interleave(grp, dim=0).contiguous()
    qt = torch.from_numpy(q).reshape(Hq, 1, d)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kh, Vh, scale=sm_scale)
    return o.reshape(Hq, d).numpy()


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("window,wl", [(0, None), (8, [8, 5]), (8, [0, 3])])
def test_d1_equals_d2(window, wl):
    c = rand_case(1, window=window, wl=wl)
    assert rel(A.decode_latent(**c), A.decode_reconstruct(**c)) < 1e-12


def test_identity_bases_equal_dense_sdpa():
    """Full rank with identity bases: the method is exactly dense GQA attention."""
    rng = np.random.default_rng(2)
    B, Hq, Hkv, d, T = 2, 28, 4, 128, 50
    D = Hkv * d
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, T, D))
    V = rng.standard_normal((B, T, D))
    eye = np.eye(D)
    kw = dict(q=q, zk=K, zv=V, bk=eye, bv=eye, lat_len=[T, 31], rank_k=D, rank_v=D,
              n_kv_heads=Hkv, sm_scale=1 / math.sqrt(d))
    for fn in (A.decode_reconstruct, A.decode_latent):
        out = fn(**kw)
        for b, L in enumerate([T, 31]):
            ref = sdpa_dense(q[b], K[b, :L], V[b, :L], Hkv, 1 / math.sqrt(d))
            assert rel(out[b], ref) < 1e-12


def test_single_token_returns_its_value():
    """T = 1: the softmax of one element is 1, so o_j = V[0, g(j)] = (Zv[0] Bv)[g(j)]."""
    c = rand_case(3, B=1, L=(1,))
    V0 = c["zv"][0, 0] @ c["bv"]
    out = A.decode_latent(**c)[0]
    for j in range(28):
        g = j // 7
        assert np.allclose(out[j], V0[g * 128:(g + 1) * 128], rtol=0, atol=1e-14)


def test_zero_query_is_mean_value():
    c = rand_case(4, B=1, L=(45,))
    c["q"][:] = 0
    V = c["zv"][0, :45] @ c["bv"]
    out = A.decode_reconstruct(**c)[0]
    for j in range(28):
        g = j // 7
        assert np.allclose(out[j], V[:, g * 128:(g + 1) * 128].mean(0), rtol=0, atol=1e-14)


def test_needle_selects_planted_token():
    """Selection bases plant one token per KV group whose score beats all others by >= 40."""
    cfg = synth.CONFIGS[0].replace(batch=2)
    li = synth.selection_needle(cfg, delta=40.0)
    args = dict(q=li.q, zk=li.zk, zv=li.zv, bk=li.bk, bv=li.bv, lat_len=li.lat_len,
                rank_k=li.rank_k, rank_v=li.rank_v, n_kv_heads=4, sm_scale=cfg.sm_scale)
    out = A.decode_latent(**args)
    bk = li.bk.double().numpy()
    bv = li.bv.double().numpy()
    zk = li.zk.double().numpy()
    zv = li.zv.double().numpy()
    for b in range(2):
        L = int(li.lat_len[b])
        K = zk[b, :L, :li.rank_k] @ bk
        V = zv[b, :L, :li.rank_v] @ bv
        for j in range(28):
            g = j // 7
            s = K[:, g * 128:(g + 1) * 128] @ li.q[b, j].double().numpy() * cfg.sm_scale
            t = int(np.argmax(s))
            assert np.sort(s)[-1] - np.sort(s)[-2] >= 40 - 1e-4   # lam is stored in float32
            assert np.allclose(out[b, j], V[t, g * 128:(g + 1) * 128], atol=L * math.exp(-40) * 10)


def test_window_only_equals_dense_attention_over_window():
    c = rand_case(5, B=2, L=(0, 0), window=16, wl=[16, 9])
    out = A.decode_reconstruct(**c)
    out2 = A.decode_latent(**c)
    for b in range(2):
        rows = [(0 + i) % 16 for i in range(c["win_len"][b])]
        ref = sdpa_dense(c["q"][b], c["kwin"][b][rows], c["vwin"][b][rows], 4, c["sm_scale"])
        assert rel(out[b], ref) < 1e-12
        assert rel(out2[b], ref) < 1e-12


def test_window_ring_slots_follow_absolute_position():
    """With L latent tokens before it, the window token at position L + i sits in slot (L+i) mod W:
    the result must equal dense attention over reconstructed rows followed by those slots."""
    c = rand_case(6, B=1, L=(13,), window=8, wl=[5])
    L = 13
    K = np.concatenate([c["zk"][0, :L] @ c["bk"], c["kwin"][0][[(L + i) % 8 for i in range(5)]]])
    V = np.concatenate([c["zv"][0, :L] @ c["bv"], c["vwin"][0][[(L + i) % 8 for i in range(5)]]])
    ref = sdpa_dense(c["q"][0], K, V, 4, c["sm_scale"])
    assert rel(A.decode_latent(**c)[0], ref) < 1e-12


def test_no_window_is_pure_latent_path():
    c = rand_case(7, window=8, wl=[0, 0])
    c0 = dict(c, window=0, kwin=None, vwin=None)
    assert rel(A.decode_latent(**c), A.decode_latent(**c0)) < 1e-15


def test_empty_sequence_is_zero():
    c = rand_case(8, L=(0, 20))
    for fn in (A.decode_reconstruct, A.decode_latent):
        out = fn(**c)
        assert np.all(out[0] == 0)
        assert np.any(out[1] != 0)


def test_token_permutation_invariance():
    c = rand_case(9, B=1, L=(64,))
    perm = np.random.default_rng(0).permutation(64)
    c2 = dict(c, zk=c["zk"][:, perm], zv=c["zv"][:, perm])
    assert rel(A.decode_reconstruct(**c2), A.decode_reconstruct(**c)) < 1e-12


def test_scale_enters_as_one_over_sqrt_d():
    """Two tokens with score difference delta: p1/p0 = exp(sm_scale * delta) exactly."""
    d, D = 128, 512
    bk = np.eye(D)[:8]
    bv = np.eye(D)[:8]
    zk = np.zeros((1, 2, 8)); zk[0, 1, 0] = 1.0
    zv = np.zeros((1, 2, 8)); zv[0, 1, 0] = 1.0     # V[1, col 0] = 1, V[0] = 0
    q = np.zeros((1, 28, d)); q[0, :, 0] = 3.0       # score(token 1) - score(token 0) = 3 * sm_scale
    out = A.decode_latent(q, zk, zv, bk, bv, [2], 8, 8, 4, 1 / math.sqrt(d))
    p1 = math.exp(3 / math.sqrt(d)) / (1 + math.exp(3 / math.sqrt(d)))
    assert abs(out[0, 0, 0] - p1) < 1e-15       # group 0 sees column 0
    assert np.all(out[0, 7:, :] == 0)            # other groups see zero columns: o = 0


tiny = st.integers(min_value=0, max_value=10_000)


@settings(max_examples=40, deadline=None)
@given(seed=tiny, Hkv=st.sampled_from([1, 2]), grp=st.sampled_from([1, 2, 3]), d=st.sampled_from([1, 2, 3]),
       rk=st.integers(1, 4), rv=st.integers(1, 4), L=st.integers(0, 4), W=st.integers(0, 3),
       wl_frac=st.integers(0, 3))
def test_bruteforce_matches_d1_d2(seed, Hkv, grp, d, rk, rv, L, W, wl_frac):
    rng = np.random.default_rng(seed)
    Hq, D = Hkv * grp, Hkv * d
    wl = min(W, wl_frac)
    q = rng.standard_normal((1, Hq, d)) * 2
    zk = rng.standard_normal((1, max(L, 1), rk))
    zv = rng.standard_normal((1, max(L, 1), rv))
    bk = rng.standard_normal((rk, D))
    bv = rng.standard_normal((rv, D))
    kw = rng.standard_normal((1, max(W, 1), D))
    vw = rng.standard_normal((1, max(W, 1), D))
    args = dict(lat_len=[L], rank_k=rk, rank_v=rv, n_kv_heads=Hkv, sm_scale=1 / math.sqrt(d),
                win_len=[wl], window=W)
    bf = np.array(A.decode_bruteforce(q.tolist(), zk.tolist(), zv.tolist(), bk.tolist(), bv.tolist(),
                                      kwin=kw.tolist(), vwin=vw.tolist(), **args))
    for fn in (A.decode_reconstruct, A.decode_latent):
        out = fn(q, zk, zv, bk, bv, kwin=kw, vwin=vw, **args)
        assert np.allclose(out, bf, rtol=1e-10, atol=1e-12)


def test_pins_catch_planted_mistakes():
    """Copies of D2 with one planted slip each must fail the dense-SDPA pin."""
    rng = np.random.default_rng(11)
    Hq, Hkv, d, T = 28, 4, 128, 20
    D = Hkv * d
    q = rng.standard_normal((Hq, d))
    Zk = rng.standard_normal((T, D))
    Zv = rng.standard_normal((T, D))
    B = np.linalg.qr(rng.standard_normal((D, D)))[0].T     # orthonormal, not symmetric
    sm = 1 / math.sqrt(d)
    ref = sdpa_dense(q, Zk @ B, Zv @ B, Hkv, sm)

    def d2(group=lambda j: j // 7, scale=sm, transpose_bk=False, drop_upproj=False, axis=0):
        out = np.zeros((Hq, d))
        Bk = B.T if transpose_bk else B
        for j in range(Hq):
            g = group(j)
            qt = q[j] @ Bk[:, g * d:(g + 1) * d].T
            s = scale * (Zk @ qt)
            p = np.exp(s - s.max()); p /= p.sum()
            a = p @ Zv
            out[j] = a[g * d:(g + 1) * d] if drop_upproj else a @ B[:, g * d:(g + 1) * d]
        return out

    assert rel(d2(), ref) < 1e-12
    q = q * 8   # sharpen the softmax so that score-path slips are visible
    ref = sdpa_dense(q, Zk @ B, Zv @ B, Hkv, sm)
    assert rel(d2(), ref) < 1e-12
    for slip in (dict(group=lambda j: j % 4), dict(scale=1.0), dict(transpose_bk=True),
                 dict(drop_upproj=True)):
        assert rel(d2(**slip), ref) > 1e-2, slip
