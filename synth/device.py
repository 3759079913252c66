"""Device staging of synthetic layer inputs (data movement only).

Copies a synth.LayerInputs to the GPU in the cache layout of the C ABI. int4 caches are
filled by the library's own bulk store (lowrank_kv_store) from the float32 latents, so no
quantisation arithmetic lives here.
"""
from __future__ import annotations

import numpy as np
import torch

import rank_kv_cache_lowrank_amd as lr

from . import LayerInputs, down_projection, projection_storage


def device_layer(li: LayerInputs, device="cuda", with_proj: bool = False):
    """Returns (lr.Model, lr.Cache) for one synthetic layer."""
    cfg = li.cfg
    model = lr.Model(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, [li.rank_k], [li.rank_v],
                     cfg.sm_scale, cfg.window, cfg.latent)
    B = cfg.batch
    lat_len = torch.from_numpy(np.asarray(li.lat_len, np.int32)).to(device)
    win_len = torch.from_numpy(np.asarray(li.win_len, np.int32)).to(device) if cfg.window else None
    kw = li.kwin.to(device) if li.kwin is not None else None
    vw = li.vwin.to(device) if li.vwin is not None else None
    pk = pv = None
    if with_proj:
        dt = torch.float32 if cfg.latent == "f32" else torch.bfloat16
        pk = projection_storage(down_projection(li.bk.double().numpy()), dt).to(device)
        pv = projection_storage(down_projection(li.bv.double().numpy()), dt).to(device)
    if cfg.latent in ("f32", "bf16"):
        cache = lr.Cache(li.zk.to(device), li.zv.to(device), li.bk.to(device), li.bv.to(device), lat_len,
                         li.t_cap, li.ld_k, li.ld_v, pk=pk, pv=pv, kwin=kw, vwin=vw, win_len=win_len)
        return model, cache
    zk, zkq = lr.latent_storage("i4g32", B, li.t_cap, li.rank_k, 0, device)
    zv, zvq = lr.latent_storage("i4g32", B, li.t_cap, li.rank_v, 0, device)
    cache = lr.Cache(zk, zv, li.bk.to(device), li.bv.to(device), lat_len, li.t_cap, 0, 0,
                     zk_qp=zkq, zv_qp=zvq, pk=pk, pv=pv, kwin=kw, vwin=vw, win_len=win_len)
    zk_rows = li.zk[:, :, :li.rank_k].contiguous().to(device)
    zv_rows = li.zv[:, :, :li.rank_v].contiguous().to(device)
    lr.lowrank_kv_store(model, 0, cache, 0, zk_rows, zv_rows)
    del zk_rows, zv_rows
    return model, cache
