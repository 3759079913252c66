"""GPU parity of the exact recent window and of per-layer rank dispatch (28-layer model with a
global rank-allocation table), against the fp64 oracle."""
import numpy as np
import pytest
import torch

import rank_kv_cache_lowrank_amd as lr
import synth
from helpers import TOL, device_layer, oracle_decode, rel_err, run_decode

pytestmark = pytest.mark.gpu
CFG4 = synth.CONFIGS[4]


def check(li, batches=None, model=None, layer=0, nsplit=0):
    m1, cache = device_layer(li)
    model = m1 if model is None else model
    mx = int(li.lat_len.max())
    out = run_decode(model, cache, li.q.cuda(), mx, nsplit=nsplit, layer=layer)
    b_list = list(range(li.cfg.batch)) if batches is None else list(batches)
    ref = oracle_decode(li, b_list)
    err = rel_err(out[b_list].numpy(), ref)
    print(f"layer={li.layer} r=({li.rank_k},{li.rank_v}) L={li.lat_len[b_list]} W={li.win_len[b_list]} "
          f"err={err:.3e}", flush=True)
    assert err <= TOL["bf16"], err
    return out


def model28(cfg):
    ranks = [synth.layer_ranks(cfg, l) for l in range(cfg.n_layers)]
    return lr.Model(cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, [r[0] for r in ranks],
                    [r[1] for r in ranks], cfg.sm_scale, cfg.window, cfg.latent)


@pytest.mark.parametrize("layer", [0, 13, 27])
def test_config4_full_size_layers_sampled(layer):
    """B=16, lengths U{2048..8192} (last 128 tokens exact), the layer's drawn ranks."""
    li = synth.make_layer(CFG4, layer)
    assert np.all(li.win_len == 128)
    check(li, batches=[0, 6, 15], model=model28(CFG4), layer=layer)


def test_all_28_layers_through_one_rank_table():
    """Every layer of the 28-layer descriptor at a reduced length: the host derives each layer's
    ranks, padding and kernel bounds from the table."""
    cfg = CFG4.replace(batch=2)
    model = model28(cfg)
    for layer in range(cfg.n_layers):
        li = synth.make_layer(cfg, layer, q_scale=16.0, lat_len=np.array([300, 77], np.int32),
                              win_len=np.array([128, 40], np.int32))
        check(li, model=model, layer=layer)


@pytest.mark.parametrize("latent,rk,rv", [("f32", 128, 96), ("i4g32", 200, 72)])
def test_window_with_other_latent_types(latent, rk, rv):
    """fp32 latents (fp32 queries: the window on the VALU workgroups of the decode kernel) and int4
    latents (the matrix-core exact-keys kernel), with partial and wrapped windows."""
    cfg = CFG4.replace(batch=4, latent=latent, rank_choices=None, rank_k=rk, rank_v=rv)
    li = synth.make_layer(cfg, 2, q_scale=16.0, lat_len=np.array([700, 130, 0, 1], np.int32),
                          win_len=np.array([128, 77, 9, 128], np.int32))
    m1, cache = device_layer(li)
    out = run_decode(m1, cache, li.q.cuda(), int(li.lat_len.max()))
    err = rel_err(out.numpy(), oracle_decode(li, list(range(4))))
    print(f"{latent} r=({rk},{rv}) err={err:.3e}", flush=True)
    assert err <= TOL[latent], err


@pytest.mark.parametrize("hq,hkv,latent", [(32, 8, "bf16"), (16, 1, "bf16"), (32, 1, "bf16"), (16, 1, "i4g32")])
def test_window_head_layouts(hq, hkv, latent):
    """Query heads per KV head 4 and 16 (the fold and the exact keys in one launch) and 32 (beyond
    that launch's bound of 16: the general exact-keys kernel, with no chunk rows)."""
    cfg = synth.Config(93, f"window-h{hq}-{hkv}", batch=3, seq_len=300, rank_k=120, rank_v=88, latent=latent,
                       window=32, n_q_heads=hq, n_kv_heads=hkv)
    li = synth.make_layer(cfg, q_scale=8.0, lat_len=np.array([300, 0, 45], np.int32),
                          win_len=np.array([32, 19, 1], np.int32))
    m1, cache = device_layer(li)
    out = run_decode(m1, cache, li.q.cuda(), int(li.lat_len.max()))
    err = rel_err(out.numpy(), oracle_decode(li, list(range(3))))
    print(f"Hq={hq} Hkv={hkv} {latent} err={err:.3e}", flush=True)
    assert err <= TOL[latent], err


def test_window_only_sequences():
    cfg = CFG4.replace(batch=5)
    li = synth.make_layer(cfg, 3, q_scale=16.0, lat_len=np.zeros(5, np.int32),
                          win_len=np.array([1, 7, 64, 127, 128], np.int32), t_cap=16)
    check(li)


def test_partial_windows_wrapping_ring():
    """Live window slots start at position L mod W and wrap around the ring."""
    cfg = CFG4.replace(batch=6)
    li = synth.make_layer(cfg, 5, q_scale=16.0, lat_len=np.array([130, 1, 255, 64, 500, 0], np.int32),
                          win_len=np.array([50, 128, 3, 128, 0, 0], np.int32))
    out = check(li, batches=[0, 1, 2, 3, 4])
    assert torch.all(out[5] == 0)


def test_sharp_scores_mixed_window_and_history():
    """Large query scale: the softmax mass moves between window and latent history per head."""
    cfg = CFG4.replace(batch=3)
    li = synth.make_layer(cfg, 9, q_scale=96.0, lat_len=np.array([1000, 2000, 17], np.int32),
                          win_len=np.array([128, 100, 128], np.int32))
    check(li)


@pytest.mark.parametrize("W", [48, 128, 200, 256])
def test_window_dead_slots_hold_nan(W):
    """Ring slots outside the live window hold NaN: the window's walk over physical slots must keep
    them out of both the scores and the values. Full windows whose live slots wrap (two runs of
    tiles that merge), partial windows inside one run or wrapping, a single slot, and W > 128 (the
    tiles are loaded when reached)."""
    import dataclasses
    cfg = CFG4.replace(batch=6, window=W, rank_choices=None, rank_k=136, rank_v=200)
    lat = np.array([3 * W + 5, 7, 0, W - 3, 1000, 2 * W - 10], np.int32)
    wl = np.array([W, W // 2, 1, W - 1, 17, 30], np.int32)
    li = synth.make_layer(cfg, 3, q_scale=16.0, lat_len=lat, win_len=wl)
    kw, vw = li.kwin.clone(), li.vwin.clone()
    for b in range(cfg.batch):
        live = {(int(lat[b]) + i) % W for i in range(int(wl[b]))}
        dead = [s for s in range(W) if s not in live]
        kw[b, dead] = float("nan")
        vw[b, dead] = float("nan")
    li = dataclasses.replace(li, kwin=kw, vwin=vw)
    out = check(li)
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("nsplit", [1, 5, 32])
def test_window_with_split_counts(nsplit):
    cfg = CFG4.replace(batch=2)
    li = synth.make_layer(cfg, 20, q_scale=16.0, lat_len=np.array([1500, 999], np.int32),
                          win_len=np.array([128, 128], np.int32))
    check(li, nsplit=nsplit)
