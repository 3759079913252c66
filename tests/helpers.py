"""Shared test plumbing: device copies of synthetic inputs, oracle arguments, error metric."""
from __future__ import annotations

import numpy as np
import torch

import synth
import rank_kv_cache_lowrank_amd as lr
from synth.device import device_layer  # noqa: F401
from oracle import attention as OA
from oracle import quant as OQ

TOL = {"f32": 5e-3, "bf16": 5e-3, "i4g32": 1e-2}


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(gpu))) if gpu.size else 0.0
    return float(np.max(np.abs(gpu - ref)) / den)


def oracle_latents(li: synth.LayerInputs, which: str, batches) -> list:
    """Stored latent values as the oracle sees them, per requested sequence (float64)."""
    z = li.zk if which == "k" else li.zv
    r = li.rank_k if which == "k" else li.rank_v
    out = []
    for b in batches:
        L = int(li.lat_len[b])
        rows = z[b, :L, :r].float().numpy()
        if li.cfg.latent == "i4g32":
            codes, s, zz = OQ.quantize_rows(rows)
            rows = OQ.dequant_rows(codes, s, zz, r)
        out.append(rows.astype(np.float64))
    return out


def oracle_decode(li: synth.LayerInputs, batches=None, fn=OA.decode_latent) -> np.ndarray:
    cfg = li.cfg
    batches = list(range(cfg.batch)) if batches is None else list(batches)
    zk = oracle_latents(li, "k", batches)
    zv = oracle_latents(li, "v", batches)
    idx = {b: i for i, b in enumerate(batches)}
    # the oracle indexes sequences by b: give it views keyed through a small adapter
    q = li.q.float().numpy()
    kw = li.kwin.float().numpy() if li.kwin is not None else None
    vw = li.vwin.float().numpy() if li.vwin is not None else None

    class ByB:
        def __init__(self, rows):
            self.rows = rows

        def __getitem__(self, b):
            return self.rows[idx[b]]

    return fn(q, ByB(zk), ByB(zv), li.bk.float().numpy(), li.bv.float().numpy(), li.lat_len,
              li.rank_k, li.rank_v, cfg.n_kv_heads, cfg.sm_scale, kwin=kw, vwin=vw,
              win_len=li.win_len, window=cfg.window, batches=batches)


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a tensor's storage (NaN patterns compare equal bit for bit)."""
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]
    return t.view(view)


def cache_snapshot(cache) -> dict:
    """Bit copies of every buffer of a cache (latents, scale/zero words, rings, lengths)."""
    return {k: bits(t).clone() for k, t in cache.tensors.items() if t is not None}


def assert_cache_unchanged(cache, snap: dict, what: str) -> None:
    for k, t in snap.items():
        assert torch.equal(bits(cache.tensors[k]), t), f"{what} modified the cache buffer {k}"


WS_CANARY = 0xA5
WS_GUARD = 4096


def guarded_workspace(n: int, device) -> tuple:
    """A workspace of n bytes followed by a canary band; returns (workspace view, full buffer)."""
    buf = torch.full((n + WS_GUARD,), WS_CANARY, dtype=torch.uint8, device=device)
    return buf[:n], buf


def assert_canary(buf: torch.Tensor, n: int, what: str) -> None:
    assert bool((buf[n:] == WS_CANARY).all()), f"{what} wrote past the end of its workspace"


def run_decode(model, cache, q, max_lat_len, nsplit=0, out_dtype=torch.float32, guard=True, layer=0):
    """Runs lowrank_attn_decode; checks guard bands around the output and past the workspace, and
    that the cache is untouched; returns out (CPU)."""
    B, Hq, d = q.shape
    n = B * Hq * d
    pad = 1024
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=out_dtype, device=q.device)
    out = buf[pad:pad + n].view(B, Hq, d)
    ws_n = lr.lowrank_attn_decode_workspace_size(model, layer, B, max_lat_len, nsplit)
    assert ws_n > 0
    ws, ws_buf = guarded_workspace(ws_n, q.device)
    snap = cache_snapshot(cache) if guard else None
    lr.lowrank_attn_decode(model, layer, cache, q, out, max_lat_len, ws, nsplit=nsplit)
    torch.cuda.synchronize()
    if guard:
        head = buf[:pad].float()
        tail = buf[pad + n:].float()
        assert torch.isnan(head).all() and torch.isnan(tail).all(), "decode wrote outside out"
        assert_canary(ws_buf, ws_n, "decode")
        assert_cache_unchanged(cache, snap, "decode")
    return out.float().cpu()
