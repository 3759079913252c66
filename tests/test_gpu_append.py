"""GPU parity of the append / bulk-store / dequant entry points against the oracle.

Bit-exact where z is exact in any summation order (identity or signed power-of-two
permutation projections, bulk store of given float32 rows); within the float32 accumulation
bound otherwise (general pseudo-inverse projection).
"""
import numpy as np
import pytest
import torch

import synth
import rank_kv_cache_lowrank_amd as lr
from oracle import append as OAP
from oracle import quant as OQ

pytestmark = pytest.mark.gpu
DEV = "cuda"


GUARD_ROWS = 3


def sentinel_storage(latent, B, t_cap, rank, ld):
    """Latent storage whose every byte starts as 0xFF (NaN for float rows and for the float16
    scale/zero words), laid out as [B][t_cap] rows followed by GUARD_ROWS spare rows; returns the
    [B, t_cap, ...] views and the flat buffers (views share their memory)."""
    if latent in ("f32", "bf16"):
        dt = torch.float32 if latent == "f32" else torch.bfloat16
        full = torch.empty(B * t_cap + GUARD_ROWS, ld, dtype=dt, device=DEV)
        full.view(torch.uint8).fill_(0xFF)
        return full[:B * t_cap].view(B, t_cap, ld), None, (full, None)
    g = (rank + 31) // 32
    codes = torch.full((B * t_cap + GUARD_ROWS, g * 16), 0xFF, dtype=torch.uint8, device=DEV)
    qp = torch.full((B * t_cap + GUARD_ROWS, g), -1, dtype=torch.int32, device=DEV)
    return codes[:B * t_cap].view(B, t_cap, g * 16), qp[:B * t_cap].view(B, t_cap, g), (codes, qp)


def assert_rows_untouched(full, B, t_cap, written):
    """Every row of a sentinel buffer outside `written` ({(b, row)}) still holds 0xFF bytes."""
    if full is None:
        return
    rows = full.view(torch.uint8).view(full.shape[0], -1)
    keep = torch.ones(rows.shape[0], dtype=torch.bool)
    for b, t in written:
        keep[b * t_cap + t] = False
    idx = torch.nonzero(keep).flatten().to(rows.device)
    assert bool((rows[idx] == 0xFF).all()), "append wrote a latent row it does not own (or past t_cap)"


def make_cache(latent, B, t_cap, rk, rv, window=0, pk=None, pv=None, D=512, lat0=0, win0=0,
               sentinel=False):
    ld_k, ld_v = synth.latent_ld(rk), synth.latent_ld(rv)
    if sentinel:
        zk, zkq, fk = sentinel_storage(latent, B, t_cap, rk, ld_k)
        zv, zvq, fv = sentinel_storage(latent, B, t_cap, rv, ld_v)
    else:
        zk, zkq = lr.latent_storage(latent, B, t_cap, rk, ld_k, DEV)
        zv, zvq = lr.latent_storage(latent, B, t_cap, rv, ld_v, DEV)
        fk = fv = (None, None)
    dt = torch.float32 if latent == "f32" else torch.bfloat16
    bk = torch.zeros(rk, D, dtype=dt, device=DEV)
    bv = torch.zeros(rv, D, dtype=dt, device=DEV)
    lat = torch.full((B,), lat0, dtype=torch.int32, device=DEV)
    win = torch.full((B,), win0, dtype=torch.int32, device=DEV) if window else None
    kw = torch.zeros(B, window, D, dtype=torch.bfloat16, device=DEV) if window else None
    vw = torch.zeros(B, window, D, dtype=torch.bfloat16, device=DEV) if window else None
    cache = lr.Cache(zk, zv, bk, bv, lat, t_cap, ld_k, ld_v, zk_qp=zkq, zv_qp=zvq, pk=pk, pv=pv,
                     kwin=kw, vwin=vw, win_len=win)
    cache.sentinel_buffers = [fk[0], fk[1], fv[0], fv[1]]
    model = lr.Model(1, 28, 4, 128, [rk], [rv], 128 ** -0.5, window, latent)
    return model, cache


def stored_rows(cache, latent, which, rank, n_rows):
    """Host copy of the stored form of rows [0, n_rows): (values) or (codes, scale16, zero16)."""
    z = cache.zk if which == "k" else cache.zv
    if latent in ("f32", "bf16"):
        return z[:, :n_rows, :rank].float().cpu().numpy()
    qp = (cache.zk_qp if which == "k" else cache.zv_qp)[:, :n_rows].cpu().numpy().view(np.uint32)
    codes = z[:, :n_rows].cpu().numpy()
    scale = (qp & 0xFFFF).astype(np.uint16).view(np.float16)
    zero = (qp >> 16).astype(np.uint16).view(np.float16)
    return codes, scale, zero


def dequant_gpu(model, cache, B, n_rows, rk, rv):
    ok = torch.empty(B, n_rows, rk, dtype=torch.float32, device=DEV)
    ov = torch.empty(B, n_rows, rv, dtype=torch.float32, device=DEV)
    lr.lowrank_kv_dequant(model, 0, cache, B, n_rows, ok, ov)
    torch.cuda.synchronize()
    return ok.cpu().numpy(), ov.cpu().numpy()


@pytest.mark.parametrize("latent", ["f32", "bf16", "i4g32"])
@pytest.mark.parametrize("rank", [358, 32, 7, 512])
def test_store_then_dequant_is_bit_exact(latent, rank):
    B, n = 3, 37
    rng = np.random.default_rng(rank)
    z = (rng.standard_normal((B, n, rank)) * (1.0 / np.sqrt(np.arange(1, rank + 1)))).astype(np.float32)
    z[0, 0, :] = 0.25                    # a degenerate group row
    model, cache = make_cache(latent, B, 64, rank, rank)
    zt = torch.from_numpy(z).to(DEV)
    lr.lowrank_kv_store(model, 0, cache, 5, zt, zt)
    torch.cuda.synchronize()
    ok, ov = dequant_gpu(model, cache, B, 5 + n, rank, rank)
    for b in range(B):
        if latent == "f32":
            ref = z[b]
        elif latent == "bf16":
            ref = OAP.bf16_rne(z[b])
        else:
            codes, s16, z16 = OQ.quantize_rows(z[b])
            ref = OQ.dequant_rows(codes, s16, z16, rank)
            got_codes, got_s, got_z = stored_rows(cache, latent, "k", rank, 5 + n)
            assert np.array_equal(got_codes[b, 5:], codes)
            assert np.array_equal(got_s[b, 5:].view(np.uint16), s16.view(np.uint16))
            assert np.array_equal(got_z[b, 5:].view(np.uint16), z16.view(np.uint16))
        assert np.array_equal(ok[b, 5:].view(np.uint32), ref.view(np.uint32))
        assert np.array_equal(ov[b, 5:].view(np.uint32), ref.view(np.uint32))


def _run_append(latent, rk, rv, P_k, P_v, xk, xv, window=0, lat0=0, win0=0, t_cap=64, with_debug=True):
    B, n_new, D = xk.shape
    dt = torch.float32 if latent == "f32" else torch.bfloat16
    pk = synth.projection_storage(P_k, dt).to(DEV)
    pv = synth.projection_storage(P_v, dt).to(DEV)
    model, cache = make_cache(latent, B, t_cap, rk, rv, window, pk, pv, D, lat0, win0)
    zdbg = torch.full((B, n_new, rk + rv), float("nan"), device=DEV) if with_debug else None
    lr.lowrank_kv_append(model, 0, cache, torch.from_numpy(xk).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(xv).to(torch.bfloat16).to(DEV), zdbg)
    torch.cuda.synchronize()
    return model, cache, (zdbg.cpu().numpy() if with_debug else None)


@pytest.mark.parametrize("latent", ["f32", "bf16", "i4g32"])
def test_append_identity_projection_bit_exact(latent):
    """r = D = 512, P = I: z = x exactly, so stored values equal the oracle's storage of x."""
    B, n_new, D = 4, 3, 512
    rng = np.random.default_rng(7)
    xk = torch.from_numpy(rng.standard_normal((B, n_new, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    xv = torch.from_numpy(rng.standard_normal((B, n_new, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    eye = np.eye(D)
    model, cache, zdbg = _run_append(latent, D, D, eye, eye, xk, xv, lat0=10)
    assert torch.all(cache.lat_len == 10 + n_new)
    assert np.array_equal(zdbg[:, :, :D], xk) and np.array_equal(zdbg[:, :, D:], xv)
    for which, x in (("k", xk), ("v", xv)):
        for b in range(B):
            ref = OAP.store_rows(x[b], latent)
            got = stored_rows(cache, latent, which, D, 10 + n_new)
            if latent == "i4g32":
                for part_got, part_ref in zip(got, ref):
                    assert np.array_equal(np.asarray(part_got)[b, 10:].view(np.uint8),
                                          np.asarray(part_ref).view(np.uint8))
            else:
                assert np.array_equal(got[b, 10:], ref)


def test_append_signed_power_of_two_permutation_bit_exact():
    """P[:, i] = +-2^e_i * unit vector: every z_i is one exact product, so z is exact."""
    B, n_new, D, r = 3, 2, 512, 358
    rng = np.random.default_rng(9)
    rows = rng.permutation(D)[:r]
    P = np.zeros((D, r))
    P[rows, np.arange(r)] = rng.choice([-1.0, 1.0], r) * 2.0 ** rng.integers(-3, 4, r)
    xk = torch.from_numpy(rng.standard_normal((B, n_new, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    xv = xk[:, ::-1].copy()
    model, cache, zdbg = _run_append("i4g32", r, r, P, P, xk, xv)
    for b in range(B):
        zk = (xk[b].astype(np.float64) @ P).astype(np.float32)
        assert np.array_equal(zdbg[b, :, :r], zk)
        codes, s16, z16 = OQ.quantize_rows(zk)
        got_codes, got_s, got_z = stored_rows(cache, "i4g32", "k", r, n_new)
        assert np.array_equal(got_codes[b], codes)
        assert np.array_equal(got_s[b].view(np.uint16), s16.view(np.uint16))
        assert np.array_equal(got_z[b].view(np.uint16), z16.view(np.uint16))


def test_append_pseudo_inverse_projection_config3_shape():
    """The int4 append leg at its benchmark shape: 16 sequences x 1 new token, P = pinv(B) in
    bf16. Two checks: the projected z (float32 accumulation) lies within the summation bound
    of the exact product, and the stored codes / scale / zero are bit-exact with the oracle's
    quantisation of that same float32 z."""
    cfg = synth.CONFIGS[3]
    r = cfg.rank_k
    B = cfg.batch
    bk = synth.to_storage(synth.gen_basis(cfg, "k", 0, r), "bf16").double().numpy()
    bv = synth.to_storage(synth.gen_basis(cfg, "v", 0, r), "bf16").double().numpy()
    Pk = torch.from_numpy(synth.down_projection(bk)).to(torch.bfloat16).double().numpy()
    Pv = torch.from_numpy(synth.down_projection(bv)).to(torch.bfloat16).double().numpy()
    xk = synth.to_storage(synth.gen_new_tokens(cfg, "k", 0, 1), "bf16").float().numpy()
    xv = synth.to_storage(synth.gen_new_tokens(cfg, "v", 0, 1), "bf16").float().numpy()
    model, cache, zdbg = _run_append("i4g32", r, r, Pk, Pv, xk, xv, lat0=20, t_cap=32)
    ok, ov = dequant_gpu(model, cache, B, 21, r, r)
    D = xk.shape[-1]
    for which, x, P, zgot, deq in (("k", xk, Pk, zdbg[:, 0, :r], ok), ("v", xv, Pv, zdbg[:, 0, r:], ov)):
        z64 = x[:, 0].astype(np.float64) @ P                      # [B, r], exact up to fp64 rounding
        bound = D * 2.0 ** -24 * (np.abs(x[:, 0]).astype(np.float64) @ np.abs(P)) + 1e-30
        assert np.all(np.abs(zgot.astype(np.float64) - z64) <= bound)
        codes, s16, z16 = OQ.quantize_rows(zgot)
        got_codes, got_s, got_z = stored_rows(cache, "i4g32", which, r, 21)
        assert np.array_equal(got_codes[:, 20], codes)
        assert np.array_equal(got_s[:, 20].view(np.uint16), s16.view(np.uint16))
        assert np.array_equal(got_z[:, 20].view(np.uint16), z16.view(np.uint16))
        ref = OQ.dequant_rows(codes, s16, z16, r)
        assert np.array_equal(deq[:, 20].view(np.uint32), ref.view(np.uint32))
        assert np.all(np.abs(ref.astype(np.float64) - z64) <= OQ.error_bound(s16, z16, r) + bound)


@pytest.mark.parametrize("n_calls", [[1] * 11, [3, 3, 2, 5], [8, 8, 1], [11], [3, 20, 2], [2, 9, 30, 1]])
def test_window_ring_matches_token_stream(n_calls):
    """Appends through an exact window W=8 from an empty sequence: window slots, lengths and the
    evicted latent rows (P = I, bf16 storage: exact) equal the oracle's token-list model, also
    for calls of more than W tokens (the call's early tokens go to the latents after the window
    tokens they push out)."""
    B, D, W = 2, 512, 8
    rng = np.random.default_rng(sum(n_calls))
    eye = np.eye(D)
    pk = torch.from_numpy(eye.astype(np.float32)).to(torch.bfloat16).to(DEV)
    model, cache = make_cache("bf16", B, 64, D, D, W, pk, pk)
    states = [OAP.SeqState(window=W, D=D) for _ in range(B)]
    total = 0
    for n in n_calls:
        xk = torch.from_numpy(rng.standard_normal((B, n, D)).astype(np.float32)).to(torch.bfloat16)
        xv = torch.from_numpy(rng.standard_normal((B, n, D)).astype(np.float32)).to(torch.bfloat16)
        lr.lowrank_kv_append(model, 0, cache, xk.to(DEV), xv.to(DEV))
        for b in range(B):
            for i in range(n):
                OAP.append_token(states[b], xk[b, i].double().numpy(), xv[b, i].double().numpy(), eye, eye)
        total += n
    torch.cuda.synchronize()
    kw = cache.kwin.float().cpu().numpy()
    vw = cache.vwin.float().cpu().numpy()
    lat = cache.lat_len.cpu().numpy()
    win = cache.win_len.cpu().numpy()
    for b in range(B):
        st = states[b]
        assert lat[b] == st.lat_len and win[b] == st.win_len
        L = st.lat_len
        for i in range(st.win_len):
            slot = (L + i) % W
            assert np.array_equal(kw[b, slot], st.ring_k[slot])
            assert np.array_equal(vw[b, slot], st.ring_v[slot])
        if L:
            got = stored_rows(cache, "bf16", "k", D, L)[b]
            assert np.array_equal(got, np.stack(st.lat_z_k).astype(np.float32))


def test_append_clamps_at_capacity():
    B, D = 2, 512
    eye = np.eye(D)
    x = np.ones((B, 3, D), np.float32)
    model, cache, _ = _run_append("bf16", D, D, eye, eye, x, x, lat0=7, t_cap=8, with_debug=False)
    assert torch.all(cache.lat_len == 8)


def _pinv_bf16(cfg, which, r):
    """The caller's down-projection of a stored bf16 basis: P = pinv(B) rounded to bf16, as float64."""
    b = synth.to_storage(synth.gen_basis(cfg, which, 0, r), "bf16").double().numpy()
    return torch.from_numpy(synth.down_projection(b)).to(torch.bfloat16).double().numpy()


def _z_bound(x, P):
    """float32-accumulation bound of z = x P over D terms: D * 2^-24 * sum |x| |P| (+ underflow slack)."""
    return x.shape[-1] * 2.0 ** -24 * (np.abs(np.asarray(x, np.float64)) @ np.abs(P)) + 1e-30


def test_append_bf16_general_projection():
    """bf16 cache, W = 0, three new tokens per sequence through a general pseudo-inverse P: z_debug
    lies within the float32 accumulation bound of the exact x P, and every stored row is the
    round-to-nearest-even bf16 of that same float32 z, bit for bit; no other row changes."""
    cfg = synth.CONFIGS[1]
    r, B, n_new, lat0, t_cap = cfg.rank_k, 4, 3, 5, 12
    Pk, Pv = _pinv_bf16(cfg, "k", r), _pinv_bf16(cfg, "v", r)
    big = cfg.replace(batch=B)
    xk = synth.to_storage(synth.gen_new_tokens(big, "k", 0, n_new), "bf16").float().numpy()
    xv = synth.to_storage(synth.gen_new_tokens(big, "v", 0, n_new), "bf16").float().numpy()
    dt = torch.bfloat16
    pk = synth.projection_storage(Pk, dt).to(DEV)
    pv = synth.projection_storage(Pv, dt).to(DEV)
    model, cache = make_cache("bf16", B, t_cap, r, r, 0, pk, pv, lat0=lat0, sentinel=True)
    zdbg = torch.full((B, n_new, 2 * r), float("nan"), device=DEV)
    lr.lowrank_kv_append(model, 0, cache, torch.from_numpy(xk).to(dt).to(DEV),
                         torch.from_numpy(xv).to(dt).to(DEV), zdbg)
    torch.cuda.synchronize()
    zdbg = zdbg.cpu().numpy()
    assert torch.all(cache.lat_len == lat0 + n_new)
    for which, x, P, zg in (("k", xk, Pk, zdbg[:, :, :r]), ("v", xv, Pv, zdbg[:, :, r:])):
        z64 = x.astype(np.float64) @ P
        assert np.all(np.abs(zg.astype(np.float64) - z64) <= _z_bound(x, P))
        got = stored_rows(cache, "bf16", which, r, lat0 + n_new)[:, lat0:]
        assert np.array_equal(got.view(np.uint32), OAP.bf16_rne(zg).view(np.uint32))
    written = {(b, lat0 + i) for b in range(B) for i in range(n_new)}
    for full in cache.sentinel_buffers:
        assert_rows_untouched(full, B, t_cap, written)


@pytest.mark.parametrize("calls", [(1, 3, 2, 1, 3, 1), (2, 13, 4)])
@pytest.mark.parametrize("latent", ["bf16", "i4g32"])
def test_window_eviction_general_projection(latent, calls):
    """An exact window W = 8 fed a token stream in calls of 1-3 tokens, or with one call longer
    than the window, with a general pseudo-inverse P: window slots and lengths equal the oracle's
    token-list model; each evicted token's z (z_debug of the call that evicted it) lies within the
    float32 accumulation bound of the oracle's x_old P; the stored row is that z's storage form
    (bf16 rounding, or the int4 codes / scale / zero), bit for bit; no other latent row and
    nothing past t_cap changes."""
    cfg = synth.CONFIGS[1]
    B, D, W, r = 3, 512, 8, 200
    t_cap = max(8, sum(calls) - W)
    Pk, Pv = _pinv_bf16(cfg, "k", r), _pinv_bf16(cfg, "v", r)
    dt = torch.bfloat16
    pk = synth.projection_storage(Pk, dt).to(DEV)
    pv = synth.projection_storage(Pv, dt).to(DEV)
    model, cache = make_cache(latent, B, t_cap, r, r, W, pk, pv, sentinel=True)
    rng = np.random.default_rng(11)
    stream_k = torch.from_numpy(rng.standard_normal((B, sum(calls), D)).astype(np.float32)).to(dt)
    stream_v = torch.from_numpy(rng.standard_normal((B, sum(calls), D)).astype(np.float32)).to(dt)
    states = [OAP.SeqState(window=W, D=D) for _ in range(B)]
    z_gpu = [[] for _ in range(B)]            # (z_k, z_v) float32 of each evicted row, in order
    pos = 0
    for n in calls:
        xk, xv = stream_k[:, pos:pos + n].contiguous(), stream_v[:, pos:pos + n].contiguous()
        before = [st.lat_len for st in states]
        zdbg = torch.full((B, n, 2 * r), float("nan"), device=DEV)
        lr.lowrank_kv_append(model, 0, cache, xk.to(DEV), xv.to(DEV), zdbg)
        torch.cuda.synchronize()
        zdbg = zdbg.cpu().numpy()
        for b in range(B):
            for i in range(n):
                OAP.append_token(states[b], xk[b, i].double().numpy(), xv[b, i].double().numpy(), Pk, Pv)
            n_ev = states[b].lat_len - before[b]
            for i in range(n_ev):
                z_gpu[b].append((zdbg[b, i, :r], zdbg[b, i, r:]))
            assert np.all(np.isnan(zdbg[b, n_ev:]))      # no z for rows the call did not write
        pos += n
    lat = cache.lat_len.cpu().numpy()
    win = cache.win_len.cpu().numpy()
    kw = cache.kwin.float().cpu().numpy()
    vw = cache.vwin.float().cpu().numpy()
    written = set()
    for b in range(B):
        st = states[b]
        assert st.lat_len == sum(calls) - W and st.win_len == W   # the oldest evicted, W in the window
        assert lat[b] == st.lat_len and win[b] == st.win_len
        for i in range(st.win_len):
            slot = (st.lat_len + i) % W
            assert np.array_equal(kw[b, slot], st.ring_k[slot])
            assert np.array_equal(vw[b, slot], st.ring_v[slot])
        for t in range(st.lat_len):                        # evicted = the oldest tokens, in order
            written.add((b, t))
            xs = (stream_k[b, t].double().numpy(), stream_v[b, t].double().numpy())
            for which, x, P, zg, z64 in (("k", xs[0], Pk, z_gpu[b][t][0], st.lat_z_k[t]),
                                         ("v", xs[1], Pv, z_gpu[b][t][1], st.lat_z_v[t])):
                assert np.all(np.abs(zg.astype(np.float64) - z64) <= _z_bound(x[None], P)[0])
                if latent == "bf16":
                    got = stored_rows(cache, "bf16", which, r, t + 1)[b, t]
                    assert np.array_equal(got.view(np.uint32), OAP.bf16_rne(zg).view(np.uint32))
                else:
                    codes, s16, z16 = OQ.quantize_rows(zg[None])
                    gc, gs, gz = stored_rows(cache, "i4g32", which, r, t + 1)
                    assert np.array_equal(gc[b, t], codes[0])
                    assert np.array_equal(gs[b, t].view(np.uint16), s16[0].view(np.uint16))
                    assert np.array_equal(gz[b, t].view(np.uint16), z16[0].view(np.uint16))
    for full in cache.sentinel_buffers:
        assert_rows_untouched(full, B, t_cap, written)
