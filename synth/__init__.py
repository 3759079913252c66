"""Seeded synthetic inputs for low-rank KV-cache decode attention.

This module is shared by the CPU oracle, the GPU tests and the benchmark.
It holds random draws, dtype casts and input construction only:

* queries q ~ N(0, 1/head_dim), optionally scaled to sharpen the softmax;
* latent rows Z[t, i] ~ N(0, 1) * i**-0.5 (i = 1..r, one-based);
* bases with orthonormal rows, from the QR factorisation of a seeded
  Gaussian (the sign of each column of Q fixed so that diag(R) > 0);
* the caller-side down-projection P = pinv(B) used by the append path;
* sequence lengths, per-layer ranks, exact-window rows and new dense K/V.

None of the method's arithmetic (query fold, scores, softmax, value
accumulation, up-projection, projection of new tokens, quantisation) lives
here; both the oracle and the HIP path compute those from these inputs.

Workloads mirror the latency setting of TraceKV ("TraceKV: Policy-Preserving
Low-Rank KV Cache Compression for Reasoning Vision-Language Models", ai4snews
page, Perspective: Qwen2.5-VL-7B-Instruct decode at batch 16, 4K-32K context)
with a Qwen2.5-VL-7B-shaped layer: 28 query heads, 4 KV heads, head_dim 128.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

# Stream ids of the seed sequence [cfg_id, stream, layer, b].
STREAM = dict(q=0, zk=1, zv=2, bk=3, bv=4, lengths=5, ranks=6, k_new=7, v_new=8,
              window=9, needle=10, perm=11, bk_next=12, bv_next=13, q_chunk=14, kv_chunk=15, spectra=16, kv_samples=17)

N_Q_HEADS = 28
N_KV_HEADS = 4
HEAD_DIM = 128
KV_WIDTH = N_KV_HEADS * HEAD_DIM


def rng(cfg_id: int, stream: str, layer: int = 0, b: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, STREAM[stream], layer, b]))


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclass(frozen=True)
class Config:
    """One workload. ``latent`` is the cache storage format: "f32", "bf16" or "i4g32"."""
    cfg_id: int
    name: str
    batch: int
    seq_len: int                 # latent tokens per sequence (configs with fixed length)
    rank_k: int
    rank_v: int
    latent: str
    n_layers: int = 1
    window: int = 0              # exact recent window W (0 = none)
    len_range: Optional[tuple] = None     # (lo, hi) inclusive: total length per sequence
    rank_choices: Optional[tuple] = None  # per-layer ranks drawn from this set
    n_append: int = 0            # new tokens per sequence for the append leg
    n_q_heads: int = N_Q_HEADS
    n_kv_heads: int = N_KV_HEADS
    head_dim: int = HEAD_DIM

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    0: Config(0, "tiny-f32-r128", batch=1, seq_len=256, rank_k=128, rank_v=128, latent="f32"),
    1: Config(1, "qwen25vl7b-bf16-r358-T4k", batch=16, seq_len=4096, rank_k=358, rank_v=358,
              latent="bf16"),
    2: Config(2, "qwen25vl7b-bf16-r256-T32k", batch=16, seq_len=32768, rank_k=256, rank_v=256,
              latent="bf16"),
    3: Config(3, "qwen25vl7b-i4g32-r358-T16k", batch=16, seq_len=16384, rank_k=358, rank_v=358,
              latent="i4g32", n_append=1),
    4: Config(4, "qwen25vl7b-28L-ragged-window128", batch=16, seq_len=0, rank_k=0, rank_v=0,
              latent="bf16", n_layers=28, window=128, len_range=(2048, 8192),
              rank_choices=tuple(range(128, 513, 8))),
}


# ----------------------------------------------------------------------------------------------
# Per-config draws
# ----------------------------------------------------------------------------------------------

def total_lengths(cfg: Config) -> np.ndarray:
    """Total tokens per sequence (latent history + exact window)."""
    if cfg.len_range is None:
        return np.full(cfg.batch, cfg.seq_len + cfg.window, dtype=np.int64)
    lo, hi = cfg.len_range
    return rng(cfg.cfg_id, "lengths").integers(lo, hi + 1, size=cfg.batch).astype(np.int64)


def split_lengths(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """(lat_len, win_len): the last ``window`` tokens of each sequence are exact and dense."""
    n = total_lengths(cfg)
    win = np.minimum(n, cfg.window)
    return (n - win).astype(np.int32), win.astype(np.int32)


def layer_ranks(cfg: Config, layer: int) -> tuple[int, int]:
    if cfg.rank_choices is None:
        return cfg.rank_k, cfg.rank_v
    ch = np.asarray(cfg.rank_choices)
    r = rng(cfg.cfg_id, "ranks", layer).integers(0, len(ch), size=2)
    return int(ch[r[0]]), int(ch[r[1]])


def latent_ld(rank: int) -> int:
    """Row stride of a stored latent row, in elements: a multiple of 8 (16-byte rows in bf16)."""
    return round_up(rank, 8)


def inv_sqrt_index(r: int) -> np.ndarray:
    """sigma_i = i**-0.5 for the one-based latent index i = 1..r."""
    return (1.0 / np.sqrt(np.arange(1, r + 1, dtype=np.float64))).astype(np.float32)


def gen_q(cfg: Config, layer: int = 0, q_scale: float = 1.0) -> np.ndarray:
    """q [B, Hq, d] float32, entries N(0, 1/d) times ``q_scale``."""
    out = np.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=np.float32)
    for b in range(cfg.batch):
        g = rng(cfg.cfg_id, "q", layer, b)
        out[b] = g.standard_normal((cfg.n_q_heads, cfg.head_dim), dtype=np.float32)
    out *= np.float32(q_scale / np.sqrt(cfg.head_dim))
    return out


def gen_latent_rows(cfg: Config, which: str, layer: int, b: int, n_rows: int, rank: int) -> np.ndarray:
    """Z[t, i] ~ N(0,1) * i**-0.5, float32 [n_rows, rank] for sequence b."""
    g = rng(cfg.cfg_id, "zk" if which == "k" else "zv", layer, b)
    z = g.standard_normal((n_rows, rank), dtype=np.float32)
    z *= inv_sqrt_index(rank)[None, :]
    return z


def gen_basis(cfg: Config, which: str, layer: int, rank: int) -> np.ndarray:
    """B [rank, D] float64 with orthonormal rows: Q^T of QR(G[D, rank]), diag(R) > 0."""
    g = rng(cfg.cfg_id, "bk" if which == "k" else "bv", layer)
    G = g.standard_normal((cfg.kv_width, rank))
    Q, R = np.linalg.qr(G)
    Q = Q * np.sign(np.diag(R))[None, :]
    return np.ascontiguousarray(Q.T)


def gen_window_rows(cfg: Config, which: str, layer: int, b: int, rank: int) -> np.ndarray:
    """Dense window rows [W, D] float32, N(0, H_r / D) with H_r = sum_{i<=r} 1/i.

    With orthonormal basis rows this is the per-component variance of a reconstructed
    row z.B when z_i ~ N(0, 1/i), so window tokens and latent-history tokens have
    comparable norms and neither side dominates the scores.
    """
    g = rng(cfg.cfg_id, "window", layer, 2 * b + (0 if which == "k" else 1))
    h = float(np.sum(1.0 / np.arange(1, rank + 1)))
    x = g.standard_normal((cfg.window, cfg.kv_width), dtype=np.float32)
    x *= np.float32(np.sqrt(h / cfg.kv_width))
    return x


def gen_new_tokens(cfg: Config, which: str, layer: int, n_new: int) -> np.ndarray:
    """Dense new K (or V) rows [B, n_new, D] float32 ~ N(0, 1)."""
    out = np.empty((cfg.batch, n_new, cfg.kv_width), dtype=np.float32)
    for b in range(cfg.batch):
        g = rng(cfg.cfg_id, "k_new" if which == "k" else "v_new", layer, b)
        out[b] = g.standard_normal((n_new, cfg.kv_width), dtype=np.float32)
    return out


def down_projection(basis_stored: np.ndarray) -> np.ndarray:
    """P = pinv(B) [D, rank] in float64, computed by the caller from the stored basis."""
    return np.linalg.pinv(np.asarray(basis_stored, dtype=np.float64))


def projection_storage(p: np.ndarray, dtype) -> torch.Tensor:
    """The library's layout of a down-projection P [D, rank]: rank-major [rank][D] (row i = P[:, i]),
    rounded once to ``dtype`` (a torch dtype)."""
    return torch.from_numpy(np.ascontiguousarray(np.asarray(p, np.float64).T, dtype=np.float32)).to(dtype).contiguous()


def gen_chunk(cfg: Config, layer: int, n_new: int, q_scale: float = 1.0, rank: Optional[int] = None):
    """A prefill chunk: q [B, n_new, Hq, d] ~ N(0, 1/d) * q_scale, and exact k, v rows
    [B, n_new, D] ~ N(0, H_r / D) (the variance of a reconstructed history row, as for the
    window rows), float32."""
    r = rank if rank is not None else layer_ranks(cfg, layer)[0]
    h = float(np.sum(1.0 / np.arange(1, r + 1)))
    q = np.empty((cfg.batch, n_new, cfg.n_q_heads, cfg.head_dim), np.float32)
    k = np.empty((cfg.batch, n_new, cfg.kv_width), np.float32)
    v = np.empty_like(k)
    for b in range(cfg.batch):
        g = rng(cfg.cfg_id, "q_chunk", layer, b)
        q[b] = g.standard_normal(q[b].shape, dtype=np.float32) * np.float32(q_scale / np.sqrt(cfg.head_dim))
        g = rng(cfg.cfg_id, "kv_chunk", layer, b)
        k[b] = g.standard_normal(k[b].shape, dtype=np.float32) * np.float32(np.sqrt(h / cfg.kv_width))
        v[b] = g.standard_normal(v[b].shape, dtype=np.float32) * np.float32(np.sqrt(h / cfg.kv_width))
    return q, k, v


def gen_kv_samples(cfg: Config, n: int, dim: int = 512, decay: float = 1.0, layer: int = 0):
    """Calibration KV rows for the weighted SVD: x = (g * s) Q^T with g ~ N(0, 1) [n, dim],
    s_k = k^(-decay/2) and Q a seeded orthogonal matrix, so the rows' spectrum decays like the
    latent index weights; and sensitivities w: 80% ~ U(0, 0.2) (insensitive states, e.g. visual
    tokens), 20% ~ U(1, 5) (sensitive ones). Returns float32 x [n, dim] and w [n]."""
    g = rng(cfg.cfg_id, "kv_samples", layer)
    q, r = np.linalg.qr(g.standard_normal((dim, dim)))
    q = q * np.sign(np.diag(r))[None, :]
    s = np.arange(1, dim + 1, dtype=np.float64) ** (-decay / 2)
    x = (g.standard_normal((n, dim)) * s[None, :]) @ q.T
    sens = g.random(n) < 0.2
    w = np.where(sens, g.uniform(1.0, 5.0, n), g.uniform(0.0, 0.2, n))
    return x.astype(np.float32), w.astype(np.float32)


def gen_spectra(cfg: Config, n_mat: int, n: int = 512) -> np.ndarray:
    """Per-matrix singular spectra [n_mat, n] float32, non-increasing: sigma_k = s * k^(-a/2)
    with a ~ U(0.3, 1.5) (how fast the energy decays) and s ~ U(0.5, 2) per matrix."""
    g = rng(cfg.cfg_id, "spectra")
    a = g.uniform(0.3, 1.5, size=n_mat)
    sc = g.uniform(0.5, 2.0, size=n_mat)
    k = np.arange(1, n + 1, dtype=np.float64)
    return (sc[:, None] * k[None, :] ** (-a[:, None] / 2)).astype(np.float32)


def gen_basis_update(cfg: Config, which: str, layer: int, old_basis: np.ndarray, rank_new: int,
                     eps: float = 0.05, stream: int = 0) -> np.ndarray:
    """A nearby new basis B' [rank_new, D] float64: the old rows (cut, or extended by fresh
    orthonormal rows), plus N(0, eps^2 / D) noise, so B' is full rank but not orthonormal."""
    old = np.asarray(old_basis, np.float64)
    D = old.shape[1]
    g = rng(cfg.cfg_id, "bk_next" if which == "k" else "bv_next", layer, stream)
    rows = old[:rank_new]
    if rank_new > old.shape[0]:
        G = g.standard_normal((D, rank_new))
        Q, R = np.linalg.qr(G)
        rows = np.concatenate([rows, (Q * np.sign(np.diag(R))[None, :]).T[old.shape[0]:]], axis=0)
    return rows + g.standard_normal((rank_new, D)) * (eps / np.sqrt(D))


def sync_projection(old_basis: np.ndarray, new_basis: np.ndarray) -> np.ndarray:
    """W = (B pinv(B'))^T [rank_new, rank] in float64, computed by the caller (as P is)."""
    return (np.asarray(old_basis, np.float64) @ np.linalg.pinv(np.asarray(new_basis, np.float64))).T


def w_storage(w: np.ndarray, latent: str, fill: float = 0.0) -> torch.Tensor:
    """W in the library's layout [rank_new][round_up(rank, 8)] and base dtype; pad = ``fill``."""
    rn, r = w.shape
    buf = np.full((rn, round_up(r, 8)), fill, np.float32)
    buf[:, :r] = w
    return to_storage(buf, "f32" if latent == "f32" else "bf16")


# ----------------------------------------------------------------------------------------------
# Storage helpers (dtype casts only)
# ----------------------------------------------------------------------------------------------

def to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round once to the storage dtype (round-to-nearest-even through torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t.clone()
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(dtype)


def padded_rows(rows: list[np.ndarray], t_cap: int, ld: int, fill: float = 0.0) -> np.ndarray:
    """Stack per-sequence [n_b, r] rows into [B, t_cap, ld] float32; unused entries = fill."""
    out = np.full((len(rows), t_cap, ld), fill, dtype=np.float32)
    for b, z in enumerate(rows):
        out[b, : z.shape[0], : z.shape[1]] = z
    return out


@dataclass
class LayerInputs:
    """One layer's inputs, in storage form (CPU tensors) plus float32 latents for int4."""
    cfg: Config
    layer: int
    rank_k: int
    rank_v: int
    ld_k: int
    ld_v: int
    t_cap: int
    q: torch.Tensor                 # [B, Hq, d] f32 (f32 latents) or bf16
    zk: torch.Tensor                # [B, t_cap, ld_k]: f32 / bf16 storage; float32 z for i4g32
    zv: torch.Tensor
    bk: torch.Tensor                # [rank_k, D] f32 or bf16
    bv: torch.Tensor
    lat_len: np.ndarray             # int32 [B]
    win_len: np.ndarray             # int32 [B]
    kwin: Optional[torch.Tensor]    # [B, W, D] bf16 ring (slot = absolute position mod W)
    vwin: Optional[torch.Tensor]


def make_layer(cfg: Config, layer: int = 0, q_scale: float = 1.0, t_cap: Optional[int] = None,
               pad_fill: float = 0.0, lat_len: Optional[np.ndarray] = None,
               win_len: Optional[np.ndarray] = None) -> LayerInputs:
    rk, rv = layer_ranks(cfg, layer)
    ll, wl = split_lengths(cfg)
    if lat_len is not None:
        ll = np.asarray(lat_len, dtype=np.int32)
    if win_len is not None:
        wl = np.asarray(win_len, dtype=np.int32)
    if t_cap is None:
        t_cap = max(int(ll.max()) if len(ll) else 0, 1)
    ld_k, ld_v = latent_ld(rk), latent_ld(rv)
    zk = padded_rows([gen_latent_rows(cfg, "k", layer, b, int(ll[b]), rk) for b in range(cfg.batch)],
                     t_cap, ld_k, pad_fill)
    zv = padded_rows([gen_latent_rows(cfg, "v", layer, b, int(ll[b]), rv) for b in range(cfg.batch)],
                     t_cap, ld_v, pad_fill)
    store = "f32" if cfg.latent in ("f32", "i4g32") else cfg.latent
    base_dtype = "f32" if cfg.latent == "f32" else "bf16"
    q = gen_q(cfg, layer, q_scale)
    kwin = vwin = None
    if cfg.window > 0:
        kw = np.zeros((cfg.batch, cfg.window, cfg.kv_width), np.float32)
        vw = np.zeros_like(kw)
        for b in range(cfg.batch):
            rows_k = gen_window_rows(cfg, "k", layer, b, rk)
            rows_v = gen_window_rows(cfg, "v", layer, b, rv)
            for i in range(int(wl[b])):
                slot = (int(ll[b]) + i) % cfg.window
                kw[b, slot] = rows_k[i]
                vw[b, slot] = rows_v[i]
        kwin, vwin = to_storage(kw, "bf16"), to_storage(vw, "bf16")
    return LayerInputs(
        cfg=cfg, layer=layer, rank_k=rk, rank_v=rv, ld_k=ld_k, ld_v=ld_v, t_cap=t_cap,
        q=to_storage(q, base_dtype), zk=to_storage(zk, store), zv=to_storage(zv, store),
        bk=to_storage(gen_basis(cfg, "k", layer, rk), base_dtype),
        bv=to_storage(gen_basis(cfg, "v", layer, rv), base_dtype),
        lat_len=ll, win_len=wl, kwin=kwin, vwin=vwin)


def selection_needle(cfg: Config, layer: int = 0, delta: float = 40.0) -> LayerInputs:
    """A needle-in-a-haystack variant built by indexing only.

    The bases select coordinates (row k of Bk is the unit vector e_{c(k)}), so for
    KV group g the latent index k_g with c(k_g) in g's columns carries that group's
    keys. Token t*_g gets Zk[t*_g, k_g] = a, every other entry of column k_g is at
    most 1 in magnitude, and every query head j of group g is lam * e (unit vector
    at column c(k_g) - 128 g), so head j's score at t*_g exceeds every other
    token's by at least sm_scale * lam * (a - 1) = ``delta``.
    """
    base = make_layer(cfg, layer)
    rk, rv = base.rank_k, base.rank_v
    D, d = cfg.kv_width, cfg.head_dim
    g = rng(cfg.cfg_id, "needle", layer)
    cols_k = g.permutation(D)[:rk]
    # make sure every group owns at least one selected column
    for grp in range(cfg.n_kv_heads):
        if not np.any((cols_k // d) == grp):
            cols_k[grp] = grp * d + int(g.integers(0, d))
    cols_v = g.permutation(D)[:rv]
    bk = np.zeros((rk, D), np.float32)
    bk[np.arange(rk), cols_k] = 1.0
    bv = np.zeros((rv, D), np.float32)
    bv[np.arange(rv), cols_v] = 1.0
    zk = base.zk.float().numpy().copy()
    zk = np.clip(zk, -1.0, 1.0)
    ll = base.lat_len
    a = 4.0
    lam = delta / (cfg.sm_scale * (a - 1.0))
    q = np.zeros((cfg.batch, cfg.n_q_heads, d), np.float32)
    grp_size = cfg.n_q_heads // cfg.n_kv_heads
    for b in range(cfg.batch):
        L = int(ll[b])
        if L == 0:
            continue
        for grp in range(cfg.n_kv_heads):
            ks = np.nonzero((cols_k // d) == grp)[0]
            k_g = int(ks[0])
            t_star = int(g.integers(0, L))
            zk[b, t_star, k_g] = a
            for j in range(grp * grp_size, (grp + 1) * grp_size):
                q[b, j, cols_k[k_g] - grp * d] = lam
    store = "f32" if cfg.latent in ("f32", "i4g32") else cfg.latent
    base_dtype = "f32" if cfg.latent == "f32" else "bf16"
    return dataclasses.replace(base, q=to_storage(q, base_dtype), zk=to_storage(zk, store),
                               bk=to_storage(bk, base_dtype), bv=to_storage(bv, base_dtype))
