"""Host-only checks of the C ABI: the library loads, exports every declared entry point, and
rejects invalid arguments before any launch (no GPU needed: these return before touching it)."""
import ctypes
import os
import re

import pytest
import torch

import rank_kv_cache_lowrank_amd as lr
from rank_kv_cache_lowrank_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lowrank_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lowrank_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = lr.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version():
    assert lr.lowrank_abi_version() == 2


# The validation tests hand the library addresses that map nothing; every case is rejected before
# a launch, but they are kept off machines with a visible GPU all the same.
host_only = pytest.mark.skipif(torch.cuda.is_available(), reason="passes unmapped device addresses")


def desc(**kw):
    base = dict(n_layers=1, n_q_heads=28, n_kv_heads=4, head_dim=128, rank_k=[358], rank_v=[358],
                sm_scale=128 ** -0.5, window=0, latent_dtype="bf16")
    base.update(kw)
    return lr.Model(**base)


def ws_size(model, layer=0, batch=16, max_len=4096, nsplit=0):
    return lr.lowrank_attn_decode_workspace_size(model, layer, batch, max_len, nsplit)


def test_workspace_size_valid_and_invalid():
    assert ws_size(desc()) > 0
    assert ws_size(desc(), layer=1) == 0                       # layer out of range
    assert ws_size(desc(n_q_heads=30)) == 0                     # 30 % 4 != 0
    assert ws_size(desc(head_dim=64)) == 0                      # unsupported head_dim
    assert ws_size(desc(rank_k=[0])) == 0
    assert ws_size(desc(rank_v=[513])) == 0
    assert ws_size(desc(), batch=-1) == 0
    assert ws_size(desc(), max_len=-5) == 0
    # more token ranges -> more partials
    assert ws_size(desc(), nsplit=64) > ws_size(desc(), nsplit=2)


def call_decode(model, cache_struct, **kw):
    lib = lr.load()
    args = dict(layer=0, batch=2, max_len=16, q=1 << 20, out=1 << 21, out_dtype=L.LR_F32, ws=1 << 22,
                ws_bytes=1 << 30, opts=None, stream=None)
    args.update(kw)
    return lib.lowrank_attn_decode(ctypes.byref(model.desc), args["layer"],
                                   ctypes.byref(cache_struct) if cache_struct is not None else None,
                                   args["batch"], args["max_len"], args["q"], args["out"], args["out_dtype"],
                                   args["ws"], args["ws_bytes"], args["opts"], args["stream"])


def fake_cache(**kw):
    c = L.lr_layer_cache()
    c.zk, c.zv = 1 << 24, 1 << 25
    c.bk, c.bv = 1 << 26, 1 << 27
    c.lat_len = 1 << 28
    c.ld_k = c.ld_v = 360
    c.t_cap = 64
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@host_only
@pytest.mark.parametrize("case,code", [
    (dict(cache=None), L.LR_EINVAL),
    (dict(cache_kw=dict(zk=None)), L.LR_EINVAL),
    (dict(cache_kw=dict(ld_k=356)), L.LR_EINVAL),             # ld < rank
    (dict(cache_kw=dict(ld_k=362)), L.LR_EINVAL),             # ld not a multiple of 8
    (dict(cache_kw=dict(zk=(1 << 24) + 4)), L.LR_EINVAL),     # misaligned latents
    (dict(max_len=65), L.LR_EINVAL),                          # max_lat_len > t_cap
    (dict(q=None), L.LR_EINVAL),
    (dict(out_dtype=7), L.LR_EINVAL),
    (dict(ws=None), L.LR_EINVAL),
    (dict(ws=(1 << 22) + 64), L.LR_EINVAL),                   # workspace not 256-aligned
    (dict(ws_bytes=16), L.LR_EWORKSPACE),
    (dict(layer=3), L.LR_EINVAL),
])
def test_decode_rejects_invalid_arguments(case, code):
    model = desc()
    cache = None if case.get("cache", 1) is None else fake_cache(**case.get("cache_kw", {}))
    kw = {k: v for k, v in case.items() if k not in ("cache", "cache_kw")}
    assert call_decode(model, cache, **kw) == code
    assert lr.lowrank_last_error() != ""


@host_only
def test_window_requires_ring_buffers():
    model = desc(window=128)
    assert call_decode(model, fake_cache()) == L.LR_EINVAL
    assert "window" in lr.lowrank_last_error()


@host_only
def test_unsupported_combinations():
    assert call_decode(desc(n_q_heads=40, n_kv_heads=4), fake_cache()) == L.LR_EUNSUPPORTED
    assert call_decode(desc(latent_dtype="f32", rank_k=[300], rank_v=[300]),
                       fake_cache(ld_k=304, ld_v=304)) == L.LR_EUNSUPPORTED


@host_only
def test_opts_reserved_fields_must_be_zero():
    o = L.lr_decode_opts()
    o.reserved[2] = 5
    assert call_decode(desc(), fake_cache(), opts=ctypes.byref(o)) == L.LR_EINVAL
    o = L.lr_decode_opts()
    o.nsplit = -1
    assert call_decode(desc(), fake_cache(), opts=ctypes.byref(o)) == L.LR_EINVAL


@host_only
def test_append_store_dequant_validation():
    lib = lr.load()
    model = desc(window=8)
    c = fake_cache(pk=1 << 29, pv=1 << 30)
    # window set but no ring
    assert lib.lowrank_kv_append(ctypes.byref(model.desc), 0, ctypes.byref(c), 2, 1, 1 << 20, 1 << 21,
                                 None, None) == L.LR_EINVAL
    model = desc()
    # n_new negative
    assert lib.lowrank_kv_append(ctypes.byref(model.desc), 0, ctypes.byref(c), 2, -1, 1 << 20, 1 << 21,
                                 None, None) == L.LR_EINVAL
    # missing projections
    c2 = fake_cache()
    assert lib.lowrank_kv_append(ctypes.byref(model.desc), 0, ctypes.byref(c2), 2, 1, 1 << 20, 1 << 21,
                                 None, None) == L.LR_EINVAL
    # store out of range
    assert lib.lowrank_kv_store(ctypes.byref(model.desc), 0, ctypes.byref(c), 2, 60, 10, 1 << 20, 1 << 21,
                                None) == L.LR_EINVAL
    # dequant beyond t_cap
    assert lib.lowrank_kv_dequant(ctypes.byref(model.desc), 0, ctypes.byref(c), 2, 65, 1 << 20, 1 << 21,
                                  None) == L.LR_EINVAL
    # int4 cache without scale/zero buffers
    m4 = desc(latent_dtype="i4g32")
    assert lib.lowrank_kv_store(ctypes.byref(m4.desc), 0, ctypes.byref(c), 2, 0, 1, 1 << 20, 1 << 21,
                                None) == L.LR_EINVAL


def call_rebase(model, src, dst, **kw):
    lib = lr.load()
    a = dict(layer=0, batch=2, max_len=16, rk_new=200, rv_new=200, wk=1 << 29, wv=1 << 30, stream=None)
    a.update(kw)
    return lib.lowrank_kv_rebase(ctypes.byref(model.desc), a["layer"],
                                 ctypes.byref(src) if src is not None else None,
                                 ctypes.byref(dst) if dst is not None else None, a["batch"], a["max_len"],
                                 a["rk_new"], a["rv_new"], a["wk"], a["wv"], a["stream"])


def fake_dst(**kw):
    c = L.lr_layer_cache()
    c.zk, c.zv = 1 << 31, 1 << 32
    c.ld_k = c.ld_v = 200
    c.t_cap = 64
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@host_only
@pytest.mark.parametrize("case,code", [
    (dict(src=None), L.LR_EINVAL),
    (dict(dst=None), L.LR_EINVAL),
    (dict(src_kw=dict(lat_len=None)), L.LR_EINVAL),
    (dict(src_kw=dict(ld_v=352)), L.LR_EINVAL),               # src ld < current rank
    (dict(dst_kw=dict(ld_k=192)), L.LR_EINVAL),               # dst ld < new rank
    (dict(dst_kw=dict(ld_v=204)), L.LR_EINVAL),               # dst ld not a multiple of 8
    (dict(dst_kw=dict(zv=(1 << 32) + 8)), L.LR_EINVAL),       # misaligned dst
    (dict(dst_kw=dict(t_cap=10)), L.LR_EINVAL),               # max_lat_len > dst t_cap
    (dict(max_len=65), L.LR_EINVAL),                          # max_lat_len > src t_cap
    (dict(rk_new=0), L.LR_EINVAL),
    (dict(rv_new=513), L.LR_EINVAL),
    (dict(wk=None), L.LR_EINVAL),
    (dict(wv=(1 << 30) + 2), L.LR_EINVAL),                    # misaligned W
    (dict(batch=-1), L.LR_EINVAL),
    (dict(layer=1), L.LR_EINVAL),
    (dict(model=dict(latent_dtype="i4g32")), L.LR_EUNSUPPORTED),
    (dict(inplace=True, dst_kw=dict(ld_k=360, ld_v=360, t_cap=32)), L.LR_EINVAL),   # in place, t_cap differs
    (dict(inplace=True, model=dict(rank_k=[512], rank_v=[512]), src_kw=dict(ld_k=512, ld_v=512),
          dst_kw=dict(ld_k=512, ld_v=512), rk_new=352, rv_new=352), L.LR_EUNSUPPORTED),  # bf16 in place, 3 W chunks
])
def test_rebase_rejects_invalid_arguments(case, code):
    model = desc(**case.get("model", {}))
    src = None if case.get("src", 1) is None else fake_cache(**case.get("src_kw", {}))
    if case.get("inplace"):
        dst = fake_cache(**case.get("dst_kw", {}))
    else:
        dst = None if case.get("dst", 1) is None else fake_dst(**case.get("dst_kw", {}))
    kw = {k: v for k, v in case.items() if k not in ("src", "dst", "src_kw", "dst_kw", "model", "inplace")}
    assert call_rebase(model, src, dst, **kw) == code
    assert lr.lowrank_last_error() != ""


@host_only
def test_rebase_zero_sizes_are_no_ops():
    assert call_rebase(desc(), fake_cache(), fake_dst(), batch=0) == L.LR_OK
    assert call_rebase(desc(), fake_cache(), fake_dst(), max_len=0) == L.LR_OK
    # in place within one W chunk, nothing to do
    assert call_rebase(desc(), fake_cache(), fake_cache(), rk_new=192, rv_new=100, batch=0) == L.LR_OK
    # rank 358 -> 352 in place: one chunk of the all-waves form
    assert call_rebase(desc(), fake_cache(), fake_cache(), rk_new=352, rv_new=352, batch=0) == L.LR_OK


@host_only
def test_zero_batch_is_a_no_op():
    # valid arguments with batch 0 return OK without launching anything
    assert call_decode(desc(), fake_cache(), batch=0) == L.LR_OK


def test_missing_library_fails_loudly(tmp_path):
    saved = L._lib
    try:
        L._lib = None
        with pytest.raises(RuntimeError):
            L.load(str(tmp_path / "missing.so"))
    finally:
        L._lib = saved


@host_only
@pytest.mark.parametrize("args,code", [
    ((4, 64, 64, 1000, 8, 64, 8), L.LR_OK),
    ((4, 64, 64, 10, 8, 64, 8), L.LR_EINVAL),        # budget below n_mat * r_min
    ((4, 64, 64, 1000, 8, 60, 8), L.LR_EINVAL),      # (r_max - r_min) % granule
    ((4, 64, 64, 1000, 0, 64, 8), L.LR_EINVAL),      # r_min < 1
    ((4, 64, 64, 1000, 8, 80, 8), L.LR_EINVAL),      # r_max > n_sigma
    ((4, 64, 32, 1000, 8, 64, 8), L.LR_EINVAL),      # sigma_ld < n_sigma
    ((0, 64, 64, 1000, 8, 64, 8), L.LR_EINVAL),      # no matrix
    ((70000, 64, 64, 10 ** 9, 8, 64, 8), L.LR_EINVAL),  # too many granules
])
def test_rank_allocate_validation(args, code):
    lib = lr.load()
    n_mat, n_sigma, ld, budget, r_min, r_max, g = args
    ws = lr.lowrank_rank_allocate_workspace_size(max(n_mat, 1), r_min, max(r_max, r_min), g)
    if code == L.LR_OK:
        # valid arguments enqueue work: only check the size query here
        assert ws >= n_mat * ((r_max - r_min) // g) * 8
        return
    assert lib.lowrank_rank_allocate(1 << 20, n_mat, n_sigma, ld, budget, r_min, r_max, g, 1 << 21, 1 << 22,
                                     1 << 30, None) == code
    assert lr.lowrank_last_error() != ""


@host_only
@pytest.mark.parametrize("args,code", [
    ((3, 1000, 512, 358, 0, L.LR_F32), L.LR_OK),
    ((0, 1000, 512, 358, 0, L.LR_F32), L.LR_EINVAL),        # no matrix
    ((3, -1, 512, 358, 0, L.LR_F32), L.LR_EINVAL),          # negative sample count
    ((3, 1000, 96, 32, 0, L.LR_F32), L.LR_EUNSUPPORTED),    # dim not a multiple of 64
    ((3, 1000, 576, 32, 0, L.LR_F32), L.LR_EUNSUPPORTED),   # dim above 512
    ((3, 1000, 512, 513, 0, L.LR_F32), L.LR_EINVAL),        # rank above dim
    ((3, 1000, 512, 0, 0, L.LR_F32), L.LR_EINVAL),          # rank below 1
    ((3, 1000, 512, 358, 65, L.LR_F32), L.LR_EINVAL),       # too many sweeps
    ((3, 1000, 512, 358, 0, L.LR_I4G32), L.LR_EINVAL),      # basis dtype
])
def test_sens_svd_batched_validation(args, code):
    """Argument checks of the batched and single-matrix weighted SVD (no work is enqueued)."""
    lib = lr.load()
    n_mat, n, dim, rank, sweeps, bdt = args
    ws = lr.lowrank_sens_svd_batched_workspace_size(n_mat, n, dim)
    if code == L.LR_OK:
        one = lr.lowrank_sens_svd_workspace_size(n, dim)
        assert one > 0 and ws == n_mat * one
        return
    assert lib.lowrank_sens_svd_batched(1 << 20, 1 << 21, n_mat, n, dim, rank, sweeps, 1 << 22, bdt, 1 << 23,
                                        1 << 24, 1 << 40, None) == code
    assert lr.lowrank_last_error() != ""
    if n_mat == 1 or n_mat == 3:
        assert lib.lowrank_sens_svd(1 << 20, 1 << 21, n, dim, rank, sweeps, 1 << 22, bdt, 1 << 23, 1 << 24,
                                    1 << 40, None) == code


@host_only
def test_sens_svd_batched_workspace_checks():
    lib = lr.load()
    ws = lr.lowrank_sens_svd_batched_workspace_size(4, 2048, 256)
    assert lib.lowrank_sens_svd_batched(1 << 20, 1 << 21, 4, 2048, 256, 64, 0, 1 << 22, L.LR_F32, 1 << 23, 1 << 24,
                                        ws - 1, None) == L.LR_EWORKSPACE
    assert lib.lowrank_sens_svd_batched(1 << 20, 1 << 21, 4, 2048, 256, 64, 0, 1 << 22, L.LR_F32, 1 << 23,
                                        (1 << 24) + 16, ws, None) == L.LR_EINVAL   # workspace alignment
    assert lr.lowrank_sens_svd_batched_workspace_size(70000, 2048, 256) == 0


def test_basis_update_workspace_size_and_rejections():
    assert lr.lowrank_basis_update_workspace_size(256, 128, 512) > 0
    assert lr.lowrank_basis_update_workspace_size(256, 128, 500) == 0       # dim not a multiple of 64
    assert lr.lowrank_basis_update_workspace_size(0, 128, 512) == 0
    assert lr.lowrank_basis_update_workspace_size(600, 0, 512) == 0         # rank > dim
    assert lr.lowrank_basis_update_workspace_size(8, -1, 512) == 0


@host_only
@pytest.mark.parametrize("kw,code", [
    (dict(dim=500), L.LR_EUNSUPPORTED),
    (dict(rank_new=0), L.LR_EINVAL),
    (dict(rank_new=385), L.LR_EINVAL),                    # > rank + n_rows
    (dict(basis_dtype=2), L.LR_EINVAL),
    (dict(basis=None), L.LR_EINVAL),
    (dict(ws_bytes=1024), L.LR_EWORKSPACE),
    (dict(sweeps=65), L.LR_EINVAL),
])
def test_basis_update_rejects_invalid_arguments(kw, code):
    lib = lr.load()
    a = dict(basis=1 << 20, basis_dtype=L.LR_BF16, sigma=1 << 21, rank=256, rows=1 << 22, n_rows=128, dim=512,
             rank_new=256, sweeps=0, basis_new=1 << 23, sigma_new=1 << 24, w=1 << 25, ws=1 << 26, ws_bytes=1 << 40)
    a.update(kw)
    rc = lib.lowrank_basis_update(a["basis"], a["basis_dtype"], a["sigma"], a["rank"], a["rows"], a["n_rows"],
                                  a["dim"], a["rank_new"], a["sweeps"], a["basis_new"], a["sigma_new"], a["w"],
                                  a["ws"], a["ws_bytes"], None)
    assert rc == code
    assert lr.lowrank_last_error() != ""
