"""lowrank_decode_step (append of one token + decode in fewer launches) against the two separate
calls: the same output bit for bit and the same cache afterwards (latent rows, rings, lengths), over
several steps, and against the oracle at the end."""
import numpy as np
import pytest
import torch

import rank_kv_cache_lowrank_amd as lr
import synth
from helpers import TOL, bits, device_layer, oracle_decode, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("latent,window", [("bf16", 0), ("bf16", 128), ("bf16", 200), ("i4g32", 0), ("i4g32", 32),
                                           ("f32", 16)])
def test_step_equals_append_then_decode(latent, window):
    base = synth.CONFIGS[4] if window else synth.CONFIGS[1]
    kw = dict(batch=5, latent=latent)
    if window:
        kw.update(window=window, rank_choices=None, rank_k=200 if latent != "f32" else 96, rank_v=136)
    else:
        kw.update(seq_len=600, rank_k=358 if latent != "f32" else 128, rank_v=358 if latent != "f32" else 128)
    cfg = base.replace(**kw)
    lat = np.array([600, 1, 0, 77, 599], np.int32)
    wl = np.array([window, window // 2, 1, window, 0], np.int32) if window else None
    li = synth.make_layer(cfg, 1 if window else 0, q_scale=16.0, lat_len=lat, win_len=wl, t_cap=620)
    model, ca = device_layer(li, with_proj=True)
    _, cb = device_layer(li, with_proj=True)
    q = li.q.cuda()
    B, D = cfg.batch, cfg.kv_width
    rng = np.random.default_rng(3)
    mx = 620
    ws_a = lr.workspace(model, 0, B, mx)
    ws_b = lr.workspace(model, 0, B, mx)
    for step in range(4):
        k_new = torch.from_numpy(rng.standard_normal((B, 1, D)).astype(np.float32)).to(torch.bfloat16).cuda()
        v_new = torch.from_numpy(rng.standard_normal((B, 1, D)).astype(np.float32)).to(torch.bfloat16).cuda()
        oa = torch.empty(B, cfg.n_q_heads, cfg.head_dim, device="cuda")
        ob = torch.empty_like(oa)
        lr.lowrank_kv_append(model, 0, ca, k_new, v_new)
        lr.lowrank_attn_decode(model, 0, ca, q, oa, mx, ws_a)
        lr.lowrank_decode_step(model, 0, cb, k_new, v_new, q, ob, mx, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), step
        for k, t in ca.tensors.items():
            if t is not None:
                assert torch.equal(bits(t), bits(cb.tensors[k])), (step, k)
    # the stepped cache against the oracle (stored latents read back, window ring as stored)
    import dataclasses
    z_k = cb.zk.cpu()
    if latent == "i4g32":
        ok = torch.empty(B, 620, cfg.rank_k, device="cuda")
        ov = torch.empty(B, 620, cfg.rank_v, device="cuda")
        lr.lowrank_kv_dequant(model, 0, cb, B, 620, ok, ov)
        torch.cuda.synchronize()
        zk, zv = ok.cpu(), ov.cpu()
        cfg_o = cfg.replace(latent="f32")
    else:
        zk, zv = z_k, cb.zv.cpu()
        cfg_o = cfg
    li2 = dataclasses.replace(li, cfg=cfg_o, zk=zk, zv=zv, lat_len=cb.lat_len.cpu().numpy(),
                              win_len=cb.win_len.cpu().numpy() if window else li.win_len,
                              kwin=cb.kwin.cpu() if window else None, vwin=cb.vwin.cpu() if window else None)
    ref = oracle_decode(li2)
    err = rel_err(ob.cpu().numpy(), ref)
    print(f"step {latent} W={window}: err vs oracle {err:.3e}", flush=True)
    assert err <= TOL[latent]
