"""lowrank_decode_step captured in a HIP graph: every replay gives the same output bits and the same
cache (latent rows, rings, lengths) as the same step run eagerly on a twin cache, with eager work
and synchronisations between the replays. The library records no memsets, only kernel launches."""
import numpy as np
import pytest
import torch

import rank_kv_cache_lowrank_amd as lr
import synth
from helpers import bits, device_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("latent,window", [("bf16", 128), ("i4g32", 0)])
def test_graph_replays_match_eager_steps(latent, window):
    base = synth.CONFIGS[4] if window else synth.CONFIGS[1]
    kw = dict(batch=6, latent=latent)
    if window:
        kw.update(window=window, rank_choices=None, rank_k=200, rank_v=136)
    else:
        kw.update(seq_len=700, rank_k=358, rank_v=358)
    cfg = base.replace(**kw)
    lat = np.array([650, 1, 0, 77, 599, 300], np.int32)
    wl = np.array([window, window // 2, 1, window, 0, 7], np.int32) if window else None
    li = synth.make_layer(cfg, 1 if window else 0, q_scale=16.0, lat_len=lat, win_len=wl, t_cap=700)
    model, ca = device_layer(li, with_proj=True)        # eager
    _, cb = device_layer(li, with_proj=True)            # graph
    q = li.q.cuda()
    B, D = cfg.batch, cfg.kv_width
    mx = 700
    ws_a = lr.workspace(model, 0, B, mx)
    ws_b = lr.workspace(model, 0, B, mx)
    k_new = torch.empty(B, 1, D, dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    oa = torch.empty(B, cfg.n_q_heads, cfg.head_dim, device="cuda")
    ob = torch.empty_like(oa)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.lowrank_decode_step(model, 0, cb, k_new, v_new, q, ob, mx, ws_b)
    rng = np.random.default_rng(4)
    for step in range(4):
        # new token rows written by eager torch work between replays (the graph reads them in place)
        k_new.copy_(torch.from_numpy(rng.standard_normal((B, 1, D)).astype(np.float32)).to(torch.bfloat16))
        v_new.copy_(torch.from_numpy(rng.standard_normal((B, 1, D)).astype(np.float32)).to(torch.bfloat16))
        lr.lowrank_decode_step(model, 0, ca, k_new, v_new, q, oa, mx, ws_a)
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(oa).all()
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), step
        for k, t in ca.tensors.items():
            if t is not None:
                assert torch.equal(bits(t), bits(cb.tensors[k])), (step, k)
        ob.fill_(float("nan"))                          # a replay must rewrite every output element
