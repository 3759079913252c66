"""ctypes binding of liblowrank_attn.so (argument marshalling only).

Function names mirror the C ABI in include/lowrank_attn.h. Tensors are PyTorch
device tensors; only their data pointers cross the boundary, together with the
current HIP stream. Every computation runs in the library's kernels; if the
library is missing this module raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# LOWRANK_ATTN_LIB selects another build of the library (e.g. a host-only sanitizer build for tests)
LIB_PATH = os.environ.get("LOWRANK_ATTN_LIB") or os.path.join(HERE, "liblowrank_attn.so")

LR_OK, LR_EINVAL, LR_EUNSUPPORTED, LR_EWORKSPACE, LR_EHIP = 0, -1, -2, -3, -4
LR_F32, LR_BF16, LR_I4G32 = 0, 1, 2
DTYPES = {"f32": LR_F32, "bf16": LR_BF16, "i4g32": LR_I4G32}

EXPORTS = ("lowrank_attn_decode_workspace_size", "lowrank_attn_decode", "lowrank_attn_decode_noalloc",
           "lowrank_attn_prefill_workspace_size",
           "lowrank_attn_prefill", "lowrank_sens_svd_workspace_size", "lowrank_sens_svd",
           "lowrank_sens_svd_batched_workspace_size", "lowrank_sens_svd_batched",
           "lowrank_rank_allocate_workspace_size", "lowrank_rank_allocate",
           "lowrank_kv_append", "lowrank_decode_step",
           "lowrank_kv_store", "lowrank_kv_dequant", "lowrank_kv_rebase", "lowrank_basis_update_workspace_size",
           "lowrank_basis_update", "lowrank_last_error",
           "lowrank_abi_version")


class LowRankError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lowrank status {code}: {msg}")
        self.code = code


class lr_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("rank_k", POINTER(c_int32)), ("rank_v", POINTER(c_int32)),
                ("sm_scale", c_float), ("window", c_int32), ("latent_dtype", c_int32)]


class lr_layer_cache(ctypes.Structure):
    _fields_ = [("zk", c_void_p), ("zv", c_void_p), ("zk_qp", c_void_p), ("zv_qp", c_void_p),
                ("bk", c_void_p), ("bv", c_void_p), ("pk", c_void_p), ("pv", c_void_p),
                ("kwin", c_void_p), ("vwin", c_void_p), ("lat_len", c_void_p), ("win_len", c_void_p),
                ("ld_k", c_int32), ("ld_v", c_int32), ("t_cap", c_int64)]


class lr_decode_opts(ctypes.Structure):
    _fields_ = [("nsplit", c_int32), ("reserved0", c_int32), ("event_begin", c_void_p),
                ("event_end", c_void_p), ("reserved", c_int32 * 4)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with rank_kv_cache_lowrank_amd.build.build()")
    lib = ctypes.CDLL(path)
    lib.lowrank_attn_decode_workspace_size.restype = c_size_t
    lib.lowrank_attn_decode_workspace_size.argtypes = [POINTER(lr_model_desc), c_int32, c_int32, c_int32,
                                                       POINTER(lr_decode_opts)]
    lib.lowrank_attn_decode.restype = c_int32
    lib.lowrank_attn_decode.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32,
                                        c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                        POINTER(lr_decode_opts), c_void_p]
    lib.lowrank_attn_decode_noalloc.restype = c_int32
    lib.lowrank_attn_decode_noalloc.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32,
                                                c_int32, c_void_p, c_void_p, c_int32, POINTER(lr_decode_opts),
                                                c_void_p]
    lib.lowrank_attn_prefill_workspace_size.restype = c_size_t
    lib.lowrank_attn_prefill_workspace_size.argtypes = [POINTER(lr_model_desc), c_int32, c_int32, c_int32,
                                                        c_int32, POINTER(lr_decode_opts)]
    lib.lowrank_attn_prefill.restype = c_int32
    lib.lowrank_attn_prefill.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32,
                                         c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                         c_void_p, c_size_t, POINTER(lr_decode_opts), c_void_p]
    lib.lowrank_sens_svd_workspace_size.restype = c_size_t
    lib.lowrank_sens_svd_workspace_size.argtypes = [c_int32, c_int32]
    lib.lowrank_sens_svd_batched_workspace_size.restype = c_size_t
    lib.lowrank_sens_svd_batched_workspace_size.argtypes = [c_int32, c_int32, c_int32]
    lib.lowrank_sens_svd_batched.restype = c_int32
    lib.lowrank_sens_svd_batched.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                             c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.lowrank_sens_svd.restype = c_int32
    lib.lowrank_sens_svd.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32,
                                     c_void_p, c_void_p, c_size_t, c_void_p]
    lib.lowrank_rank_allocate_workspace_size.restype = c_size_t
    lib.lowrank_rank_allocate_workspace_size.argtypes = [c_int32, c_int32, c_int32, c_int32]
    lib.lowrank_rank_allocate.restype = c_int32
    lib.lowrank_rank_allocate.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int64, c_int32, c_int32, c_int32,
                                          c_void_p, c_void_p, c_size_t, c_void_p]
    lib.lowrank_kv_append.restype = c_int32
    lib.lowrank_kv_append.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32,
                                      c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.lowrank_decode_step.restype = c_int32
    lib.lowrank_decode_step.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_size_t,
                                        POINTER(lr_decode_opts), c_void_p]
    lib.lowrank_kv_store.restype = c_int32
    lib.lowrank_kv_store.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32,
                                     c_int64, c_int64, c_void_p, c_void_p, c_void_p]
    lib.lowrank_kv_dequant.restype = c_int32
    lib.lowrank_kv_dequant.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache), c_int32,
                                       c_int64, c_void_p, c_void_p, c_void_p]
    lib.lowrank_kv_rebase.restype = c_int32
    lib.lowrank_kv_rebase.argtypes = [POINTER(lr_model_desc), c_int32, POINTER(lr_layer_cache),
                                      POINTER(lr_layer_cache), c_int32, c_int32, c_int32, c_int32, c_void_p,
                                      c_void_p, c_void_p]
    lib.lowrank_basis_update_workspace_size.restype = c_size_t
    lib.lowrank_basis_update_workspace_size.argtypes = [c_int32, c_int32, c_int32]
    lib.lowrank_basis_update.restype = c_int32
    lib.lowrank_basis_update.argtypes = [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                                         c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.lowrank_last_error.restype = ctypes.c_char_p
    lib.lowrank_last_error.argtypes = []
    lib.lowrank_abi_version.restype = c_int32
    lib.lowrank_abi_version.argtypes = []
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(code: int) -> None:
    if code != LR_OK:
        raise LowRankError(code, lowrank_last_error())


class Model:
    """lr_model_desc plus the host rank tables it points to."""

    def __init__(self, n_layers: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 rank_k: Sequence[int], rank_v: Sequence[int], sm_scale: float, window: int,
                 latent_dtype: str):
        self._rk = (c_int32 * n_layers)(*[int(r) for r in rank_k])
        self._rv = (c_int32 * n_layers)(*[int(r) for r in rank_v])
        self.desc = lr_model_desc(n_layers, n_q_heads, n_kv_heads, head_dim,
                                  ctypes.cast(self._rk, POINTER(c_int32)),
                                  ctypes.cast(self._rv, POINTER(c_int32)),
                                  float(sm_scale), window, DTYPES[latent_dtype])
        self.latent_dtype = latent_dtype
        self.n_q_heads, self.n_kv_heads, self.head_dim = n_q_heads, n_kv_heads, head_dim
        self.window = window
        self.rank_k = [int(r) for r in rank_k]
        self.rank_v = [int(r) for r in rank_v]


class Cache:
    """lr_layer_cache over torch tensors (the tensors are kept alive by this object)."""

    def __init__(self, zk, zv, bk, bv, lat_len, t_cap: int, ld_k: int = 0, ld_v: int = 0,
                 zk_qp=None, zv_qp=None, pk=None, pv=None, kwin=None, vwin=None, win_len=None):
        self.tensors = dict(zk=zk, zv=zv, zk_qp=zk_qp, zv_qp=zv_qp, bk=bk, bv=bv, pk=pk, pv=pv,
                            kwin=kwin, vwin=vwin, lat_len=lat_len, win_len=win_len)
        self.t_cap = int(t_cap)
        self.ld_k, self.ld_v = int(ld_k), int(ld_v)
        self.refresh()

    def refresh(self) -> None:
        t = self.tensors
        self.c = lr_layer_cache(_ptr(t["zk"]), _ptr(t["zv"]), _ptr(t["zk_qp"]), _ptr(t["zv_qp"]),
                                _ptr(t["bk"]), _ptr(t["bv"]), _ptr(t["pk"]), _ptr(t["pv"]),
                                _ptr(t["kwin"]), _ptr(t["vwin"]), _ptr(t["lat_len"]), _ptr(t["win_len"]),
                                self.ld_k, self.ld_v, self.t_cap)

    def __getattr__(self, name):
        tensors = self.__dict__.get("tensors")
        if tensors is not None and name in tensors:
            return tensors[name]
        raise AttributeError(name)


def _opts(nsplit: int, events=None):
    if not nsplit and events is None:
        return None
    o = lr_decode_opts()
    o.nsplit = int(nsplit)
    if events is not None:
        o.event_begin, o.event_end = events
    return ctypes.byref(o)


# ---- the C ABI, one Python function per entry point --------------------------------------------

def lowrank_abi_version() -> int:
    return int(load().lowrank_abi_version())


def lowrank_last_error() -> str:
    return load().lowrank_last_error().decode("utf-8", "replace")


def lowrank_attn_decode_workspace_size(model: Model, layer: int, batch: int, max_lat_len: int,
                                       nsplit: int = 0) -> int:
    return int(load().lowrank_attn_decode_workspace_size(ctypes.byref(model.desc), layer, batch,
                                                         max_lat_len, _opts(nsplit)))


def lowrank_attn_decode(model: Model, layer: int, cache: Cache, q: torch.Tensor, out: torch.Tensor,
                        max_lat_len: int, workspace: torch.Tensor, nsplit: int = 0, stream=None,
                        events=None) -> None:
    """events: optional (begin, end) raw hipEvent_t handles recorded around the latent kernel."""
    out_dtype = LR_F32 if out.dtype == torch.float32 else LR_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_attn_decode(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), q.shape[0],
                                      max_lat_len, _ptr(q), _ptr(out), out_dtype, _ptr(workspace), ws_bytes,
                                      _opts(nsplit, events), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20   # LOWRANK_NOALLOC_SCRATCH_BYTES


def lowrank_attn_decode_noalloc(model: Model, layer: int, cache: Cache, q: torch.Tensor, out: torch.Tensor,
                                max_lat_len: int, nsplit: int = 0, stream=None, events=None) -> None:
    """lowrank_attn_decode through the library's own device scratch (no workspace argument)."""
    out_dtype = LR_F32 if out.dtype == torch.float32 else LR_BF16
    _check(load().lowrank_attn_decode_noalloc(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), q.shape[0],
                                              max_lat_len, _ptr(q), _ptr(out), out_dtype, _opts(nsplit, events),
                                              _stream(stream)))


def lowrank_attn_prefill_workspace_size(model: Model, layer: int, batch: int, n_new: int, max_lat_len: int,
                                        nsplit: int = 0) -> int:
    return int(load().lowrank_attn_prefill_workspace_size(ctypes.byref(model.desc), layer, batch, n_new,
                                                          max_lat_len, _opts(nsplit)))


def lowrank_attn_prefill(model: Model, layer: int, cache: Cache, q: torch.Tensor, k_new: torch.Tensor,
                         v_new: torch.Tensor, out: torch.Tensor, max_lat_len: int, workspace: torch.Tensor,
                         nsplit: int = 0, stream=None, events=None) -> None:
    """q [B][n_new][Hq][d], k_new/v_new [B][n_new][D], out [B][n_new][Hq][d]."""
    out_dtype = LR_F32 if out.dtype == torch.float32 else LR_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_attn_prefill(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), q.shape[0],
                                       q.shape[1], max_lat_len, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
                                       out_dtype, _ptr(workspace), ws_bytes, _opts(nsplit, events),
                                       _stream(stream)))


def prefill_workspace(model: Model, layer: int, batch: int, n_new: int, max_lat_len: int, nsplit: int = 0,
                      device="cuda") -> torch.Tensor:
    n = lowrank_attn_prefill_workspace_size(model, layer, batch, n_new, max_lat_len, nsplit)
    if n == 0:
        raise LowRankError(LR_EINVAL, "workspace size query rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def lowrank_sens_svd_workspace_size(n_samples: int, dim: int) -> int:
    return int(load().lowrank_sens_svd_workspace_size(n_samples, dim))


def lowrank_sens_svd(x: torch.Tensor, w: torch.Tensor, rank: int, basis: torch.Tensor, sigma: torch.Tensor,
                     workspace: torch.Tensor, sweeps: int = 0, stream=None) -> None:
    """x [n][dim] bf16, w [n] f32; basis [rank][dim] f32 or bf16 (output), sigma [dim] f32 (output)."""
    n, dim = x.shape
    bdt = LR_F32 if basis.dtype == torch.float32 else LR_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_sens_svd(_ptr(x), _ptr(w), n, dim, rank, sweeps, _ptr(basis), bdt, _ptr(sigma),
                                   _ptr(workspace), ws_bytes, _stream(stream)))


def lowrank_sens_svd_batched_workspace_size(n_mat: int, n_samples: int, dim: int) -> int:
    return int(load().lowrank_sens_svd_batched_workspace_size(n_mat, n_samples, dim))


def lowrank_sens_svd_batched(x: torch.Tensor, w: torch.Tensor, rank: int, basis: torch.Tensor, sigma: torch.Tensor,
                             workspace: torch.Tensor, sweeps: int = 0, stream=None) -> None:
    """x [n_mat][n][dim] bf16, w [n_mat][n] f32; basis [n_mat][rank][dim] f32 or bf16 (output), sigma
    [n_mat][dim] f32 (output)."""
    n_mat, n, dim = x.shape
    bdt = LR_F32 if basis.dtype == torch.float32 else LR_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_sens_svd_batched(_ptr(x), _ptr(w), n_mat, n, dim, rank, sweeps, _ptr(basis), bdt,
                                           _ptr(sigma), _ptr(workspace), ws_bytes, _stream(stream)))


def lowrank_rank_allocate_workspace_size(n_mat: int, r_min: int, r_max: int, granule: int) -> int:
    return int(load().lowrank_rank_allocate_workspace_size(n_mat, r_min, r_max, granule))


def lowrank_rank_allocate(sigma: torch.Tensor, budget: int, r_min: int, r_max: int, granule: int,
                          ranks: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """sigma [n_mat][n] float32 (row stride = its row length), ranks [n_mat] int32 output."""
    n_mat, n = sigma.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_rank_allocate(_ptr(sigma), n_mat, n, sigma.stride(0), budget, r_min, r_max, granule,
                                        _ptr(ranks), _ptr(workspace), ws_bytes, _stream(stream)))


def lowrank_kv_append(model: Model, layer: int, cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor,
                      z_debug: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(load().lowrank_kv_append(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), k_new.shape[0],
                                    k_new.shape[1], _ptr(k_new), _ptr(v_new), _ptr(z_debug), _stream(stream)))


def lowrank_decode_step(model: Model, layer: int, cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor,
                        q: torch.Tensor, out: torch.Tensor, max_lat_len: int, workspace: torch.Tensor,
                        nsplit: int = 0, stream=None, events=None) -> None:
    """lowrank_kv_append of one token per sequence (k_new, v_new [B][1][D]) then lowrank_attn_decode."""
    out_dtype = LR_F32 if out.dtype == torch.float32 else LR_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_decode_step(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), q.shape[0],
                                      _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), out_dtype, max_lat_len,
                                      _ptr(workspace), ws_bytes, _opts(nsplit, events), _stream(stream)))


def lowrank_kv_store(model: Model, layer: int, cache: Cache, row0: int, zk_rows: torch.Tensor,
                     zv_rows: torch.Tensor, stream=None) -> None:
    _check(load().lowrank_kv_store(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), zk_rows.shape[0],
                                   row0, zk_rows.shape[1], _ptr(zk_rows), _ptr(zv_rows), _stream(stream)))


def lowrank_kv_dequant(model: Model, layer: int, cache: Cache, batch: int, n_rows: int, zk_out: torch.Tensor,
                       zv_out: torch.Tensor, stream=None) -> None:
    _check(load().lowrank_kv_dequant(ctypes.byref(model.desc), layer, ctypes.byref(cache.c), batch, n_rows,
                                     _ptr(zk_out), _ptr(zv_out), _stream(stream)))


def lowrank_kv_rebase(model: Model, layer: int, src: Cache, dst: Cache, max_lat_len: int, rank_k_new: int,
                      rank_v_new: int, wk: torch.Tensor, wv: torch.Tensor, stream=None) -> None:
    """wk [rank_k_new][round_up(rank_k, 8)], wv likewise: W = (B pinv(B'))^T in the base dtype."""
    _check(load().lowrank_kv_rebase(ctypes.byref(model.desc), layer, ctypes.byref(src.c), ctypes.byref(dst.c),
                                    src.zk.shape[0], max_lat_len, rank_k_new, rank_v_new, _ptr(wk), _ptr(wv),
                                    _stream(stream)))


def lowrank_basis_update_workspace_size(rank: int, n_rows: int, dim: int) -> int:
    return int(load().lowrank_basis_update_workspace_size(rank, n_rows, dim))


def lowrank_basis_update(basis: torch.Tensor, sigma: torch.Tensor, rows: Optional[torch.Tensor], rank_new: int,
                         basis_new: torch.Tensor, sigma_new: torch.Tensor, w: torch.Tensor, workspace: torch.Tensor,
                         sweeps: int = 0, stream=None) -> None:
    """basis [rank][dim] f32 or bf16, sigma [rank] f32, rows [n][dim] bf16 (or None); outputs basis_new
    [rank_new][dim] (basis dtype), sigma_new [rank_new] f32, w [rank_new][round_up(rank, 8)] (basis dtype)."""
    rank, dim = basis.shape
    n = 0 if rows is None else rows.shape[0]
    bdt = LR_F32 if basis.dtype == torch.float32 else LR_BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().lowrank_basis_update(_ptr(basis), bdt, _ptr(sigma), rank, _ptr(rows), n, dim, rank_new, sweeps,
                                       _ptr(basis_new), _ptr(sigma_new), _ptr(w), _ptr(workspace), ws_bytes,
                                       _stream(stream)))


# ---- device memory plumbing ---------------------------------------------------------------------

def workspace(model: Model, layer: int, batch: int, max_lat_len: int, nsplit: int = 0,
              device="cuda") -> torch.Tensor:
    n = lowrank_attn_decode_workspace_size(model, layer, batch, max_lat_len, nsplit)
    if n == 0:
        raise LowRankError(LR_EINVAL, "workspace size query rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def latent_storage(latent: str, batch: int, t_cap: int, rank: int, ld: int, device="cuda"):
    """Allocates one latent matrix in the cache format: (values, scale/zero words or None)."""
    if latent == "f32":
        return torch.zeros(batch, t_cap, ld, dtype=torch.float32, device=device), None
    if latent == "bf16":
        return torch.zeros(batch, t_cap, ld, dtype=torch.bfloat16, device=device), None
    groups = (rank + 31) // 32
    return (torch.zeros(batch, t_cap, groups * 16, dtype=torch.uint8, device=device),
            torch.zeros(batch, t_cap, groups, dtype=torch.int32, device=device))
