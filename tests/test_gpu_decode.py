"""GPU parity of lowrank_attn_decode against the fp64 oracle (max|gpu-ref|/max|ref| gates:
5e-3 for fp32/bf16 latents, 1e-2 for int4)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import synth
from helpers import TOL, device_layer, oracle_decode, rel_err, run_decode

pytestmark = pytest.mark.gpu


def check(li, batches=None, nsplit=0, max_lat_len=None, out_dtype=torch.float32, tol=None):
    model, cache = device_layer(li)
    q = li.q.cuda()
    mx = int(li.lat_len.max()) if max_lat_len is None else max_lat_len
    out = run_decode(model, cache, q, mx, nsplit=nsplit, out_dtype=out_dtype)
    b_list = list(range(li.cfg.batch)) if batches is None else list(batches)
    ref = oracle_decode(li, b_list)
    err = rel_err(out[b_list].numpy(), ref)
    t = TOL[li.cfg.latent] if tol is None else tol
    print(f"cfg={li.cfg.name} B={li.cfg.batch} r=({li.rank_k},{li.rank_v}) nsplit={nsplit} err={err:.3e}",
          flush=True)
    assert err <= t, err
    return out, ref


@pytest.mark.parametrize("q_scale", [1.0, 32.0])
def test_config0_tiny_f32(q_scale):
    check(synth.make_layer(synth.CONFIGS[0], q_scale=q_scale))


def test_config0_needle():
    check(synth.selection_needle(synth.CONFIGS[0]))


def test_config1_full_size_sampled():
    """B=16, T=4096, r=358 bf16 in the launch configuration the benchmark uses."""
    li = synth.make_layer(synth.CONFIGS[1])
    check(li, batches=[0, 7, 15])


def test_config2_full_size_sampled():
    """B=16, T=32768, r=256 bf16: long context, many token ranges."""
    li = synth.make_layer(synth.CONFIGS[2])
    check(li, batches=[0, 15])


@pytest.mark.parametrize("q_scale", [32.0, 128.0])
def test_config1_sharp_reduced(q_scale):
    cfg = synth.CONFIGS[1].replace(batch=4, seq_len=1000)
    check(synth.make_layer(cfg, q_scale=q_scale))


def test_config2_needle_reduced():
    cfg = synth.CONFIGS[2].replace(batch=3, seq_len=2000)
    check(synth.selection_needle(cfg))


@pytest.mark.parametrize("nsplit", [1, 2, 7, 16, 64])
def test_split_invariance(nsplit):
    cfg = synth.CONFIGS[1].replace(batch=3, seq_len=2100)
    li = synth.make_layer(cfg, q_scale=32.0)
    out, _ = check(li, nsplit=nsplit)
    ref_out, _ = check(li, nsplit=3)
    # both meet the oracle gate; their mutual difference is held to the same bar
    assert rel_err(out.numpy(), ref_out.numpy()) <= TOL["bf16"]


@pytest.mark.parametrize("latent", ["bf16", "i4g32"])
def test_balanced_ranges_extreme_raggedness(latent):
    """Ragged lengths take balanced ranges (planned on the device from the lengths): one long
    sequence gets up to twice the uniform count of ranges, tiny and empty ones none or one. Every
    sequence against the oracle, an explicit split count (uniform ranges) as a second reference,
    and a max_lat_len above every length."""
    cfg = synth.CONFIGS[1].replace(batch=12, seq_len=4100, latent=latent)
    lens = np.array([4100, 1, 0, 16, 17, 3000, 5, 2500, 0, 33, 4095, 64], np.int32)
    li = synth.make_layer(cfg, q_scale=16.0, lat_len=lens, t_cap=4100)
    out, _ = check(li, max_lat_len=4100)
    assert torch.all(out[2] == 0) and torch.all(out[8] == 0)
    uni, _ = check(li, nsplit=7, max_lat_len=4100)
    assert rel_err(out.numpy(), uni.numpy()) <= TOL[latent]


def test_ragged_lengths_and_empty_sequences():
    cfg = synth.CONFIGS[1].replace(batch=8, seq_len=300)
    lens = np.array([0, 1, 31, 32, 33, 200, 299, 300], np.int32)
    li = synth.make_layer(cfg, q_scale=32.0, lat_len=lens, t_cap=300)
    out, _ = check(li, batches=list(range(1, 8)))
    assert torch.all(out[0] == 0)


def test_lengths_below_max_and_ragged_tail():
    cfg = synth.CONFIGS[2].replace(batch=5, seq_len=3000)
    lens = np.array([3000, 2999, 1500, 77, 2048], np.int32)
    li = synth.make_layer(cfg, q_scale=32.0, lat_len=lens, t_cap=3000)
    check(li)


@pytest.mark.parametrize("rank", [1, 16, 33, 100, 128, 255, 256, 300, 358, 384, 448, 500, 512])
def test_rank_sweep(rank):
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=97, rank_k=rank, rank_v=rank)
    check(synth.make_layer(cfg, q_scale=32.0))


def test_unequal_ranks():
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=150, rank_k=136, rank_v=504)
    check(synth.make_layer(cfg, q_scale=32.0))
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=150, rank_k=512, rank_v=128)
    check(synth.make_layer(cfg, q_scale=32.0))


def test_nan_in_pad_columns_is_ignored():
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=200)
    li = synth.make_layer(cfg, q_scale=32.0, pad_fill=float("nan"), t_cap=256)
    # rows past lat_len are NaN too (pad_fill covers them)
    assert torch.isnan(li.zk.float()).any()
    check(li)


def test_nan_query_head_stays_confined():
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=200)
    li = synth.make_layer(cfg, q_scale=32.0)
    li.q[1, 5, 3] = float("nan")
    model, cache = device_layer(li)
    out = run_decode(model, cache, li.q.cuda(), 200)
    assert torch.isnan(out[1, 5]).all()
    mask = torch.ones(2, 28, dtype=torch.bool)
    mask[1, 5] = False
    assert not torch.isnan(out[mask]).any()


@pytest.mark.parametrize("latent", ["bf16", "i4g32"])
def test_bf16_output(latent):
    """bf16 output = the float32 result rounded to nearest even, bit for bit (the same kernels
    compute both), and the float32 result meets the latent type's gate. Against the oracle each
    bf16 element is then within gate * max|ref| + half a bf16 ulp of the float32 value
    (<= 2^-8 |o|): the rounding of the output itself is storage, not the computation."""
    cfg = synth.CONFIGS[1 if latent == "bf16" else 3].replace(batch=3, seq_len=500)
    li = synth.make_layer(cfg, q_scale=32.0)
    o32, ref = check(li)
    model, cache = device_layer(li)
    o16 = run_decode(model, cache, li.q.cuda(), int(li.lat_len.max()), out_dtype=torch.bfloat16)
    assert torch.equal(o16.to(torch.bfloat16).view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    bound = TOL[latent] * np.max(np.abs(ref)) + 2.0 ** -8 * np.abs(o32.numpy().astype(np.float64))
    assert np.all(np.abs(o16.numpy().astype(np.float64) - ref) <= bound)


def test_deterministic():
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=700)
    li = synth.make_layer(cfg, q_scale=32.0)
    model, cache = device_layer(li)
    q = li.q.cuda()
    a = run_decode(model, cache, q, 700)
    b = run_decode(model, cache, q, 700)
    assert torch.equal(a, b)


def test_max_len_zero_gives_zero():
    cfg = synth.CONFIGS[1].replace(batch=2, seq_len=64)
    li = synth.make_layer(cfg, lat_len=np.zeros(2, np.int32), t_cap=64)
    model, cache = device_layer(li)
    out = run_decode(model, cache, li.q.cuda(), 0)
    assert torch.all(out == 0)


# ---- int4 latents (groups of 32, fp16 scale and zero): dequantised in-kernel -----------------

def test_config3_full_size_sampled():
    """B=16, T=16384, r=358 int4 (12 groups, the last with 6 live indices)."""
    li = synth.make_layer(synth.CONFIGS[3])
    check(li, batches=[0, 9, 15])


@pytest.mark.parametrize("q_scale", [1.0, 32.0, 128.0])
def test_int4_reduced(q_scale):
    cfg = synth.CONFIGS[3].replace(batch=3, seq_len=1200)
    check(synth.make_layer(cfg, q_scale=q_scale))


@pytest.mark.parametrize("rank", [1, 7, 31, 32, 33, 40, 64, 100, 200, 256, 300, 384, 448, 500, 512])
def test_int4_rank_sweep(rank):
    cfg = synth.CONFIGS[3].replace(batch=2, seq_len=97, rank_k=rank, rank_v=rank)
    check(synth.make_layer(cfg, q_scale=32.0))


def test_int4_unequal_ranks():
    cfg = synth.CONFIGS[3].replace(batch=2, seq_len=333, rank_k=72, rank_v=488)
    check(synth.make_layer(cfg, q_scale=32.0))
    cfg = synth.CONFIGS[3].replace(batch=2, seq_len=333, rank_k=504, rank_v=40)
    check(synth.make_layer(cfg, q_scale=32.0))


def test_int4_needle():
    cfg = synth.CONFIGS[3].replace(batch=2, seq_len=3000)
    check(synth.selection_needle(cfg))


@pytest.mark.parametrize("nsplit", [1, 7, 64])
def test_int4_split_invariance(nsplit):
    cfg = synth.CONFIGS[3].replace(batch=2, seq_len=2500)
    li = synth.make_layer(cfg, q_scale=32.0)
    out, _ = check(li, nsplit=nsplit)
    ref_out, _ = check(li, nsplit=3)
    assert rel_err(out.numpy(), ref_out.numpy()) <= TOL["i4g32"]


def test_int4_ragged_lengths_and_empty():
    cfg = synth.CONFIGS[3].replace(batch=6, seq_len=400)
    lens = np.array([0, 1, 15, 16, 17, 400], np.int32)
    li = synth.make_layer(cfg, q_scale=32.0, lat_len=lens, t_cap=400)
    out, _ = check(li, batches=list(range(1, 6)))
    assert torch.all(out[0] == 0)


def test_int4_folded_query_beyond_fp16_range():
    """A selection needle whose folded query entries (~8e4) exceed the fp16 range: the per-head
    power-of-two scale keeps them representable and the one-hot softmax picks the needle."""
    cfg = synth.CONFIGS[3].replace(batch=2, seq_len=700)
    check(synth.selection_needle(cfg, delta=40.0 * 4096))


def test_int4_with_exact_window():
    cfg = synth.CONFIGS[4].replace(batch=3, latent="i4g32")
    li = synth.make_layer(cfg, 11, q_scale=16.0, lat_len=np.array([900, 33, 0], np.int32),
                          win_len=np.array([128, 60, 5], np.int32))
    check(li)


@pytest.mark.parametrize("latent", ["bf16", "i4g32"])
def test_resume_from_saved_cache_is_bitwise_identical(latent):
    """Checkpoint / resume: every buffer of a layer cache (latents, scale/zero words, window rings,
    lengths) saved with torch.save and loaded back with weights_only=True gives a decode output equal
    bit for bit to the original cache's, and so does the next append + decode on both."""
    import io

    import rank_kv_cache_lowrank_amd as lr

    cfg = synth.CONFIGS[4].replace(batch=3, latent=latent, rank_choices=None, rank_k=200, rank_v=136)
    li = synth.make_layer(cfg, 1, q_scale=16.0, lat_len=np.array([500, 37, 0], np.int32),
                          win_len=np.array([128, 90, 3], np.int32), t_cap=520)
    model, cache = device_layer(li, with_proj=True)
    names = [k for k, t in cache.tensors.items() if t is not None]
    blob = io.BytesIO()
    torch.save({k: cache.tensors[k].cpu() for k in names}, blob)
    blob.seek(0)
    loaded = torch.load(blob, weights_only=True)
    t = {k: loaded[k].to("cuda") for k in names}
    cache2 = lr.Cache(t["zk"], t["zv"], t["bk"], t["bv"], t["lat_len"], cache.t_cap, cache.ld_k, cache.ld_v,
                      zk_qp=t.get("zk_qp"), zv_qp=t.get("zv_qp"), pk=t.get("pk"), pv=t.get("pv"),
                      kwin=t.get("kwin"), vwin=t.get("vwin"), win_len=t.get("win_len"))
    q = li.q.cuda()
    mx = int(li.lat_len.max()) + 4
    a = run_decode(model, cache, q, mx)
    b = run_decode(model, cache2, q, mx)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    rng = np.random.default_rng(5)
    for n in (1, 3):
        k_new = torch.from_numpy(rng.standard_normal((3, n, 512)).astype(np.float32)).to(torch.bfloat16).cuda()
        v_new = torch.from_numpy(rng.standard_normal((3, n, 512)).astype(np.float32)).to(torch.bfloat16).cuda()
        lr.lowrank_kv_append(model, 0, cache, k_new, v_new)
        lr.lowrank_kv_append(model, 0, cache2, k_new, v_new)
        a = run_decode(model, cache, q, mx)
        b = run_decode(model, cache2, q, mx)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    for k in names:
        assert torch.equal(cache.tensors[k].view(torch.uint8), cache2.tensors[k].view(torch.uint8)), k


@pytest.mark.parametrize("latent,rank", [("bf16", 358), ("bf16", 512), ("i4g32", 358)])
@pytest.mark.parametrize("vscale", [1e4, 1e-6])
@pytest.mark.parametrize("nsplit", [0, 7])
def test_value_partials_far_from_unit_scale(latent, rank, vscale, nsplit):
    """The token ranges' value partials of bf16 and int4 latents are stored as fp16 with a power
    of two per (range, head) folded into the range's (m, l). Value latents scaled by 1e4 make the
    unscaled partials overflow fp16 (a range sums up to 2^8 times its tokens' values, since the
    reference max moves lazily), and by 1e-6 push them into fp16's subnormals; both must still
    meet the oracle gate. Rank 512 takes the layout in which two waves hold each head's value
    blocks (they agree on one power of two through LDS); automatic (balanced) and explicit splits."""
    cfg = synth.CONFIGS[1].replace(batch=3, seq_len=3000, latent=latent, rank_k=rank, rank_v=rank)
    li = synth.make_layer(cfg, q_scale=8.0)
    li = dataclasses.replace(li, zv=(li.zv.float() * vscale).to(li.zv.dtype))
    check(li, nsplit=nsplit)
