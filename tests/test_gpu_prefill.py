"""GPU parity of lowrank_attn_prefill (chunked prefill attention) against the oracle (P2, on the
same stored inputs), at the decode tolerances: 5e-3 (fp32/bf16 latents), 1e-2 (int4)."""
import numpy as np
import pytest
import torch

import synth
import rank_kv_cache_lowrank_amd as lr
from helpers import (TOL, assert_cache_unchanged, assert_canary, cache_snapshot, device_layer, guarded_workspace,
                     oracle_latents, rel_err)
from oracle import prefill as OP

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_prefill(model, cache, q, k, v, max_len, nsplit=0, out_dtype=torch.float32):
    B, C, Hq, d = q.shape
    n = q.numel()
    pad = 1024
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=out_dtype, device=DEV)
    out = buf[pad:pad + n].view(B, C, Hq, d)
    ws_n = lr.lowrank_attn_prefill_workspace_size(model, 0, B, C, max_len, nsplit)
    assert ws_n > 0
    ws, ws_buf = guarded_workspace(ws_n, DEV)
    snap = cache_snapshot(cache)
    lr.lowrank_attn_prefill(model, 0, cache, q, k, v, out, max_len, ws, nsplit=nsplit)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[pad + n:].float()).all(), \
        "prefill wrote outside out"
    assert_canary(ws_buf, ws_n, "prefill")
    assert_cache_unchanged(cache, snap, "prefill")
    return out.float().cpu().numpy()


def chunk_inputs(cfg, C, q_scale=1.0, rank=None):
    q, k, v = synth.gen_chunk(cfg, 0, C, q_scale, rank)
    qdt = "f32" if cfg.latent == "f32" else "bf16"
    return (synth.to_storage(q, qdt).to(DEV), synth.to_storage(k, "bf16").to(DEV),
            synth.to_storage(v, "bf16").to(DEV))


def oracle(li, q, k, v, batches=None):
    cfg = li.cfg
    batches = list(range(cfg.batch)) if batches is None else list(batches)
    zk = oracle_latents(li, "k", batches)
    zv = oracle_latents(li, "v", batches)
    idx = {b: i for i, b in enumerate(batches)}

    class ByB:
        def __init__(self, rows):
            self.rows = rows

        def __getitem__(self, b):
            return self.rows[idx[b]]

    kw = li.kwin.float().numpy() if li.kwin is not None else None
    vw = li.vwin.float().numpy() if li.vwin is not None else None
    return OP.prefill_latent(q.float().cpu().numpy(), ByB(zk), ByB(zv), li.bk.float().numpy(),
                             li.bv.float().numpy(), li.lat_len, li.rank_k, li.rank_v, cfg.n_kv_heads,
                             cfg.sm_scale, k.float().cpu().numpy(), v.float().cpu().numpy(), kwin=kw, vwin=vw,
                             win_len=li.win_len, window=cfg.window, batches=batches)


def small(latent, rank, B=3, L=(0, 37, 300), window=0, wl=None, t_cap=None):
    cfg = synth.Config(90, f"prefill-{latent}-r{rank}", batch=B, seq_len=max(L), rank_k=rank, rank_v=rank,
                       latent=latent, window=window)
    li = synth.make_layer(cfg, lat_len=np.asarray(L, np.int32), t_cap=t_cap,
                          win_len=None if wl is None else np.asarray(wl, np.int32))
    return cfg, li


@pytest.mark.parametrize("latent,rank,C", [("bf16", 358, 8), ("bf16", 256, 5), ("bf16", 64, 17),
                                           ("f32", 128, 6), ("i4g32", 358, 4), ("bf16", 512, 3)])
def test_prefill_matches_oracle(latent, rank, C):
    cfg, li = small(latent, rank)
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, C, rank=rank)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()))
    ref = oracle(li, q, k, v)
    assert rel_err(out, ref) < TOL[latent]


@pytest.mark.parametrize("latent,rank", [("bf16", 358), ("i4g32", 200), ("f32", 128)])
def test_prefill_one_token_chunk(latent, rank):
    """A chunk of one token per sequence, with a window: the token's own row is among its keys
    (unlike a decode step, where the new token is already stored)."""
    cfg, li = small(latent, rank, L=(120, 0, 33), window=16, wl=(16, 5, 0))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 1)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()))
    assert rel_err(out, oracle(li, q, k, v)) < TOL[latent]


@pytest.mark.parametrize("q_scale", [32.0, 128.0])
def test_prefill_sharp_queries(q_scale):
    cfg, li = small("bf16", 256, L=(200, 64, 1))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 6, q_scale)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()))
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


@pytest.mark.parametrize("latent,rank", [("bf16", 358), ("f32", 128), ("i4g32", 200)])
def test_prefill_with_exact_window(latent, rank):
    """Window slots and the chunk's own rows as exact keys: the dedicated bf16 kernels, the
    matrix-core exact-keys kernel beside the decode kernels (int4), the VALU workgroups (fp32)."""
    cfg, li = small(latent, rank, L=(120, 0, 33), window=16, wl=(16, 5, 0))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 7)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()))
    assert rel_err(out, oracle(li, q, k, v)) < TOL[latent]


@pytest.mark.parametrize("nsplit", [1, 3, 16])
def test_prefill_split_invariance(nsplit):
    cfg, li = small("bf16", 358, L=(500, 77, 260))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 4)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()), nsplit=nsplit)
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


def test_prefill_bf16_output_and_empty_cache():
    cfg, li = small("bf16", 128, L=(0, 0, 5))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 3)
    out = run_prefill(model, cache, q, k, v, 5, out_dtype=torch.bfloat16)
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]
    # the first token of an empty sequence attends to itself only: its own value rows
    vv = v.float().cpu().numpy()
    for j in range(28):
        g = j // 7
        np.testing.assert_allclose(out[0, 0, j], vv[0, 0, g * 128:(g + 1) * 128], rtol=1e-2, atol=1e-3)


def test_chunk_then_append_then_next_chunk():
    """Prefill a chunk, store it with lowrank_kv_append (projection + storage), prefill the next
    chunk: the second chunk sees the first one's stored latents (read back exactly) as history."""
    C = 8
    cfg, li = small("bf16", 256, L=(40, 3, 100), t_cap=100 + C)
    model, cache = device_layer(li, with_proj=True)
    q1, k1, v1 = chunk_inputs(cfg, C)
    run_prefill(model, cache, q1, k1, v1, int(li.lat_len.max()))
    lr.lowrank_kv_append(model, 0, cache, k1, v1)
    torch.cuda.synchronize()
    lat2 = cache.lat_len.cpu().numpy()
    np.testing.assert_array_equal(lat2, li.lat_len + C)
    T2 = int(lat2.max())
    ok = torch.empty(cfg.batch, T2, li.rank_k, dtype=torch.float32, device=DEV)
    ov = torch.empty(cfg.batch, T2, li.rank_v, dtype=torch.float32, device=DEV)
    lr.lowrank_kv_dequant(model, 0, cache, cfg.batch, T2, ok, ov)
    q2 = q1.flip(1).contiguous()
    k2 = (k1 * 0.5).contiguous()
    v2 = (-v1).contiguous()
    out = run_prefill(model, cache, q2, k2, v2, T2)
    zk = ok.cpu().numpy()
    zv = ov.cpu().numpy()
    ref = OP.prefill_latent(q2.float().cpu().numpy(), zk, zv, li.bk.float().numpy(), li.bv.float().numpy(), lat2,
                            li.rank_k, li.rank_v, cfg.n_kv_heads, cfg.sm_scale, k2.float().cpu().numpy(),
                            v2.float().cpu().numpy())
    assert rel_err(out, ref) < TOL["bf16"]


def test_prefill_long_chunk_and_full_window():
    """Exact keys over several staged tiles (128 window slots + a 40-token chunk) and several
    64-row blocks per KV head (40 tokens x 7 heads)."""
    cfg, li = small("bf16", 256, L=(50, 300, 17), window=128, wl=(128, 100, 0))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 40)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()))
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


@pytest.mark.parametrize("first_tile_score", [-40.0, -100.0])
@pytest.mark.parametrize("long_ranges", [False, True])
def test_prefill_low_first_tile(first_tile_score, long_ranges):
    """The first 16 latent rows of sequences 0 and 1 are set to one row z solving q~ . z = target
    (base-2 score units) for every chunk token and head at once (least norm; 168 equations in 358
    unknowns). The later tiles then lead the first tile's max by about -target: -40 stays on the
    single pass (p up to 2^40), -100 sends the workgroups through the exact-max passes. The later
    scores are unchanged, so the softmax stays as well conditioned as the plain case. With
    long_ranges, one range per sequence of more than 4096 tokens: the layout with both head blocks
    in one wave."""
    cfg, li = small("bf16", 358, L=(4500, 4200, 17) if long_ranges else (300, 64, 17))
    C = 6
    q, k, v = chunk_inputs(cfg, C, rank=358)
    qn = q.float().cpu().numpy()
    bk = li.bk.float().numpy().reshape(358, cfg.n_kv_heads, 128)
    grp = cfg.n_q_heads // cfg.n_kv_heads
    to_base2 = cfg.sm_scale * 1.4426950408889634
    for b in (0, 1):
        qt = np.stack([qn[b, :, h] @ bk[:, h // grp].T for h in range(cfg.n_q_heads)], 1).reshape(-1, 358)
        z = np.linalg.lstsq(qt, np.full(qt.shape[0], first_tile_score / to_base2), rcond=None)[0]
        li.zk[b, :16, :358] = torch.from_numpy(np.tile(z, (16, 1))).to(li.zk.dtype)
    model, cache = device_layer(li)
    out = run_prefill(model, cache, q, k, v, int(li.lat_len.max()), nsplit=1 if long_ranges else 0)
    assert np.isfinite(out).all()
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


@pytest.mark.parametrize("rank,C", [(358, 5), (256, 9), (512, 2)])
def test_prefill_long_ranges(rank, C):
    """Token ranges of more than 4096 tokens (one per sequence) take the latent kernel's layout
    with both head blocks in one wave, short ranges the one with a head block per wave: both
    against the oracle."""
    cfg, li = small("bf16", rank, B=2, L=(5000, 4200))
    q, k, v = chunk_inputs(cfg, C, rank=rank)
    model, cache = device_layer(li)
    ref = oracle(li, q, k, v)
    for nsplit in (1, 8):                   # 5000-token ranges, then 625-token ranges
        out = run_prefill(model, cache, q, k, v, 5000, nsplit=nsplit)
        assert rel_err(out, ref) < TOL["bf16"], nsplit


@pytest.mark.parametrize("rank", [358, 100])
def test_prefill_tile_pairs(rank):
    """Latent lengths of 1 to 5 tiles of 16 rows, full and ragged, one range per sequence: the
    latent kernel runs the value products of two tiles at once (K = 32 tokens) and a lone last
    tile on its own when the count is odd."""
    cfg, li = small("bf16", rank, B=8, L=(1, 16, 17, 32, 33, 48, 64, 79))
    q, k, v = chunk_inputs(cfg, 5, rank=rank)
    model, cache = device_layer(li)
    ref = oracle(li, q, k, v)
    for nsplit in (1, 3):
        out = run_prefill(model, cache, q, k, v, 79, nsplit=nsplit)
        assert rel_err(out, ref) < TOL["bf16"], nsplit


@pytest.mark.parametrize("rank_k,rank_v", [(358, 400), (400, 358), (450, 512)])
def test_prefill_unequal_ranks_ring_depths(rank_k, rank_v):
    """Unequal key and value ranks give the latent kernel 5-stage rings (one barrier per pair of
    tiles with the shallowest lookahead that allows) and 4-stage rings (one barrier per tile);
    long single ranges of odd and even tile counts and ragged ends, against the oracle."""
    cfg = synth.Config(93, f"prefill-r{rank_k}-{rank_v}", batch=3, seq_len=500, rank_k=rank_k, rank_v=rank_v,
                       latent="bf16")
    li = synth.make_layer(cfg, lat_len=np.asarray([500, 77, 264], np.int32))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 5)
    ref = oracle(li, q, k, v)
    for nsplit in (1, 2):
        out = run_prefill(model, cache, q, k, v, 500, nsplit=nsplit)
        assert rel_err(out, ref) < TOL["bf16"], nsplit


@pytest.mark.parametrize("rank", [358, 512])
@pytest.mark.parametrize("vscale", [1e4, 1e-6])
@pytest.mark.parametrize("nsplit", [0, 1])
def test_prefill_value_partials_far_from_unit_scale(rank, vscale, nsplit):
    """The latent kernel stores each (chunk token, range, head) value partial as fp16 with a power
    of two folded into its (m, l). Value latents scaled by 1e4 would overflow unscaled fp16
    partials and by 1e-6 push them into the subnormals; both must meet the oracle gate, with
    several ranges per sequence and with one range of more than 4096 tokens (the layout with
    both head blocks in one wave)."""
    cfg, li = small("bf16", rank, B=2, L=(4500, 1300))
    li.zv.mul_(vscale)
    q, k, v = chunk_inputs(cfg, 6, rank=rank)
    model, cache = device_layer(li)
    out = run_prefill(model, cache, q, k, v, 4500, nsplit=nsplit)
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


@pytest.mark.parametrize("rank", [358, 100])
def test_prefill_nan_pad_columns(rank):
    """Stored rows whose pad columns (past the rank, inside the last 16-byte granule) hold NaN:
    they must not reach the scores."""
    cfg = synth.Config(91, f"prefill-nanpad-r{rank}", batch=2, seq_len=90, rank_k=rank, rank_v=rank,
                       latent="bf16")
    li = synth.make_layer(cfg, lat_len=np.asarray([90, 33], np.int32), pad_fill=float("nan"))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 9, rank=rank)
    out = run_prefill(model, cache, q, k, v, 90)
    assert np.isfinite(out).all()
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 1), (32, 1)])
def test_prefill_head_layouts(hq, hkv):
    """Query heads per KV head 4 and 16 (the dedicated bf16 prefill kernels) and 32 (beyond their
    bound of 16: the decode kernels over the chunk's query tokens), with a window."""
    cfg = synth.Config(92, f"prefill-h{hq}-{hkv}", batch=2, seq_len=150, rank_k=100, rank_v=100, latent="bf16",
                       window=8, n_q_heads=hq, n_kv_heads=hkv)
    li = synth.make_layer(cfg, lat_len=np.asarray([150, 41], np.int32), win_len=np.asarray([8, 3], np.int32))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 9, rank=100)
    out = run_prefill(model, cache, q, k, v, 150)
    assert rel_err(out, oracle(li, q, k, v)) < TOL["bf16"]


def test_full_size_sampled():
    """16 sequences x 4096 latent rows at rank 358 (bf16) and a 32-token chunk, sampled sequences."""
    cfg = synth.CONFIGS[1]
    li = synth.make_layer(cfg)
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 32)
    out = run_prefill(model, cache, q, k, v, cfg.seq_len)
    batches = [0, 7, 15]
    ref = oracle(li, q, k, v, batches)
    assert rel_err(out[batches], ref) < TOL["bf16"]


def test_invalid_arguments():
    cfg, li = small("bf16", 64, L=(4, 4, 4))
    model, cache = device_layer(li)
    q, k, v = chunk_inputs(cfg, 2)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = lr.prefill_workspace(model, 0, 3, 2, 4)
    with pytest.raises(lr.LowRankError):
        lr.lowrank_attn_prefill(model, 0, cache, q, k, v, out, 4, ws[:16])
    assert lr.lowrank_attn_prefill_workspace_size(model, 0, 3, 0, 4) == 0
    assert lr.lowrank_attn_prefill_workspace_size(model, 0, 65536, 1, 4) == 0
