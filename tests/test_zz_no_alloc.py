"""The allocation-free decode entry point (lowrank_attn_decode_noalloc) against lowrank_attn_decode.

Both run the same kernels, the first through the library's per-GPU device scratch array, the second
through a caller workspace, so the outputs must agree bit for bit. Two calls in a row (the second
with a smaller batch, context and rank than the first, so stale scratch contents from the first
call are present) for each latent type, one with an exact window; and a request larger than the
array is rejected before any launch.
"""
import numpy as np
import pytest
import torch

import rank_kv_cache_lowrank_amd as lr
import synth
from helpers import device_layer, oracle_decode, rel_err, TOL

pytestmark = pytest.mark.gpu


def _both(li):
    model, cache = device_layer(li)
    q = li.q.cuda()
    B = li.cfg.batch
    mx = int(li.lat_len.max())
    ref = torch.empty(B, li.cfg.n_q_heads, li.cfg.head_dim, dtype=torch.float32, device="cuda")
    ws = lr.workspace(model, 0, B, mx)
    lr.lowrank_attn_decode(model, 0, cache, q, ref, mx, ws)
    pad = 256
    n = ref.numel()
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[pad:pad + n].view_as(ref)
    assert lr.lowrank_attn_decode_workspace_size(model, 0, B, mx) <= lr.NOALLOC_SCRATCH_BYTES
    lr.lowrank_attn_decode_noalloc(model, 0, cache, q, out, mx)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[pad + n:]).all()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    return out.cpu()


@pytest.mark.parametrize("latent", ["bf16", "i4g32", "f32"])
def test_noalloc_equals_workspace_decode_two_calls(latent):
    big = synth.CONFIGS[1].replace(batch=16, seq_len=3000, latent=latent,
                                   rank_k=256 if latent == "f32" else 358, rank_v=256 if latent == "f32" else 358)
    small = big.replace(batch=5, seq_len=700, rank_k=136, rank_v=200)
    for cfg, lens in ((big, None), (small, np.array([700, 0, 13, 699, 350], np.int32))):
        li = synth.make_layer(cfg, q_scale=32.0, lat_len=lens, t_cap=cfg.seq_len)
        out = _both(li)
        ref = oracle_decode(li, [0, cfg.batch - 1])
        err = rel_err(out[[0, cfg.batch - 1]].numpy(), ref)
        print(f"noalloc {latent} B={cfg.batch} T={cfg.seq_len} err={err:.3e}", flush=True)
        assert err <= TOL[latent]


def test_noalloc_with_window_two_calls():
    cfg = synth.CONFIGS[4].replace(batch=6)
    li = synth.make_layer(cfg, 3, q_scale=16.0)
    _both(li)
    li2 = synth.make_layer(cfg.replace(batch=2), 7, q_scale=16.0, lat_len=np.array([500, 3], np.int32),
                           win_len=np.array([128, 9], np.int32))
    _both(li2)


def test_noalloc_rejects_requests_beyond_the_scratch_array():
    """2048 sequences at rank 512: the per-range partials alone exceed the array, so the call
    returns LR_EWORKSPACE and launches nothing (out keeps its contents)."""
    B, T, r = 2048, 64, 512
    model = lr.Model(1, 28, 4, 128, [r], [r], 128 ** -0.5, 0, "bf16")
    need = lr.lowrank_attn_decode_workspace_size(model, 0, B, T)
    assert need > lr.NOALLOC_SCRATCH_BYTES
    z = torch.zeros(B, T, r, dtype=torch.bfloat16, device="cuda")
    basis = torch.zeros(r, 512, dtype=torch.bfloat16, device="cuda")
    lat = torch.full((B,), T, dtype=torch.int32, device="cuda")
    cache = lr.Cache(z, z, basis, basis, lat, T, r, r)
    q = torch.zeros(B, 28, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, 28, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(lr.LowRankError) as e:
        lr.lowrank_attn_decode_noalloc(model, 0, cache, q, out, T)
    assert e.value.code == lr.LR_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
