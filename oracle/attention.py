"""Decode attention over a low-rank latent KV cache: plain float64 definitions.

TEST INFRASTRUCTURE ONLY (see the package header).

Method (TraceKV abstract: attention reads "low-dimensional latents of KV
states"; iS-KV abstract: an exact recent window sits beside the latent
history). For one layer and one sequence b with L latent tokens and W_b exact
window tokens:

    K = Zk[:L] @ Bk            V = Zv[:L] @ Bv           (reconstructed keys/values, [L, D])
    K += window keys           V += window values        (row-wise concatenation)
    for query head j with KV head g = j // (Hq / Hkv):
        s_t  = sm_scale * q_j . K[t, g*d:(g+1)*d]
        p    = softmax(s)
        o_j  = sum_t p_t V[t, g*d:(g+1)*d]

A sequence with no tokens at all has output 0 (the softmax is undefined there).

Functions
---------
``decode_reconstruct``  D1: the definition above, written out (primary oracle).
``decode_latent``       D2: the same result computed in latent space, as the
                        library does: fold q into the latent space, score the
                        latent keys, accumulate latent values, up-project.
``decode_bruteforce``   D3: D1 in pure-Python loops for tiny shapes.

Pins (tests/test_oracle.py): D1 = D2 to 1e-12; full rank with identity bases
equals torch's scaled_dot_product_attention; T=1, q=0, needle and
window-only closed forms; permutation invariance; D3 on random tiny shapes.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().float().numpy()
    return np.asarray(x, dtype=np.float64)


def window_rows(win: np.ndarray, lat_len: int, win_len: int, window: int) -> np.ndarray:
    """Live rows of an exact-window ring: absolute positions lat_len .. lat_len+win_len-1,
    slot = position mod window."""
    if window == 0 or win_len == 0:
        return np.zeros((0, win.shape[-1] if win is not None else 0))
    slots = [(lat_len + i) % window for i in range(win_len)]
    return win[slots]


def _softmax(s: np.ndarray, axis: int = 0) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def decode_reconstruct(q, zk, zv, bk, bv, lat_len: Sequence[int], rank_k: int, rank_v: int,
                       n_kv_heads: int, sm_scale: float, kwin=None, vwin=None,
                       win_len: Optional[Sequence[int]] = None, window: int = 0,
                       batches: Optional[Sequence[int]] = None) -> np.ndarray:
    """D1: reconstruct K and V from the latents, then plain softmax attention.

    q [B, Hq, d]; zk [B, >=L, >=rank_k] and zv [B, >=L, >=rank_v] hold the stored
    latent values (dequantised already for int4 caches); bk [>=rank_k, D], bv
    [>=rank_v, D]; kwin/vwin [B, W, D] rings. Returns float64 [len(batches), Hq, d].
    """
    q = _f64(q)
    bk = _f64(bk)[:rank_k]
    bv = _f64(bv)[:rank_v]
    B, Hq, d = q.shape
    grp = Hq // n_kv_heads
    batches = range(B) if batches is None else batches
    out = np.zeros((len(batches), Hq, d))
    for i, b in enumerate(batches):
        L = int(lat_len[b])
        K = _f64(zk[b][:L])[:, :rank_k] @ bk
        V = _f64(zv[b][:L])[:, :rank_v] @ bv
        if window:
            wl = int(win_len[b])
            K = np.concatenate([K, window_rows(_f64(kwin[b]), L, wl, window)], axis=0)
            V = np.concatenate([V, window_rows(_f64(vwin[b]), L, wl, window)], axis=0)
        if K.shape[0] == 0:
            continue
        for g in range(n_kv_heads):
            heads = slice(g * grp, (g + 1) * grp)
            Kg = K[:, g * d:(g + 1) * d]
            Vg = V[:, g * d:(g + 1) * d]
            s = sm_scale * (Kg @ q[b, heads].T)           # [T, grp]
            p = _softmax(s, axis=0)
            out[i, heads] = p.T @ Vg
    return out


def decode_latent(q, zk, zv, bk, bv, lat_len: Sequence[int], rank_k: int, rank_v: int,
                  n_kv_heads: int, sm_scale: float, kwin=None, vwin=None,
                  win_len: Optional[Sequence[int]] = None, window: int = 0,
                  batches: Optional[Sequence[int]] = None) -> np.ndarray:
    """D2: the latent-domain computation, step by step, in float64.

    1. fold:       qt_j = q_j @ Bk[:, g*d:(g+1)*d]^T                     [rank_k]
    2. scores:     s_t  = sm_scale * Zk[t] . qt_j   (latent tokens)
                   s_w  = sm_scale * q_j . Kwin[w, g]  (window tokens)
    3. softmax over the union of latent and window tokens
    4. accumulate: A_j  = sum_t p_t Zv[t]                                [rank_v]
    5. up-project: o_j  = A_j @ Bv[:, g*d:(g+1)*d] + sum_w p_w Vwin[w, g]
    """
    q = _f64(q)
    bk = _f64(bk)[:rank_k]
    bv = _f64(bv)[:rank_v]
    B, Hq, d = q.shape
    grp = Hq // n_kv_heads
    batches = range(B) if batches is None else batches
    out = np.zeros((len(batches), Hq, d))
    for i, b in enumerate(batches):
        L = int(lat_len[b])
        Zk = _f64(zk[b][:L])[:, :rank_k]
        Zv = _f64(zv[b][:L])[:, :rank_v]
        if window:
            wl = int(win_len[b])
            Kw = window_rows(_f64(kwin[b]), L, wl, window)
            Vw = window_rows(_f64(vwin[b]), L, wl, window)
        else:
            Kw = np.zeros((0, bk.shape[1]))
            Vw = np.zeros((0, bv.shape[1]))
        if L + Kw.shape[0] == 0:
            continue
        for g in range(n_kv_heads):
            heads = slice(g * grp, (g + 1) * grp)
            cols = slice(g * d, (g + 1) * d)
            qt = q[b, heads] @ bk[:, cols].T                # [grp, rank_k]
            s_lat = sm_scale * (Zk @ qt.T)                   # [L, grp]
            s_win = sm_scale * (Kw[:, cols] @ q[b, heads].T)  # [Wb, grp]
            p = _softmax(np.concatenate([s_lat, s_win], axis=0), axis=0)
            A = p[:L].T @ Zv                                 # [grp, rank_v]
            out[i, heads] = A @ bv[:, cols] + p[L:].T @ Vw[:, cols]
    return out


def decode_bruteforce(q, zk, zv, bk, bv, lat_len, rank_k, rank_v, n_kv_heads, sm_scale,
                      kwin=None, vwin=None, win_len=None, window=0):
    """D3: D1 with nested Python loops and math.exp only (tiny shapes).

    All arguments are nested Python lists (or anything indexable); returns nested lists.
    """
    B = len(q)
    Hq = len(q[0])
    d = len(q[0][0])
    D = len(bk[0])
    grp = Hq // n_kv_heads
    out = []
    for b in range(B):
        L = int(lat_len[b])
        keys, vals = [], []
        for t in range(L):
            keys.append([sum(float(zk[b][t][i]) * float(bk[i][c]) for i in range(rank_k)) for c in range(D)])
            vals.append([sum(float(zv[b][t][i]) * float(bv[i][c]) for i in range(rank_v)) for c in range(D)])
        if window:
            for w in range(int(win_len[b])):
                slot = (L + w) % window
                keys.append([float(x) for x in kwin[b][slot]])
                vals.append([float(x) for x in vwin[b][slot]])
        ob = []
        for j in range(Hq):
            g = j // grp
            if not keys:
                ob.append([0.0] * d)
                continue
            s = [sm_scale * sum(float(q[b][j][c]) * k[g * d + c] for c in range(d)) for k in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = sum(e)
            ob.append([sum(e[t] / tot * vals[t][g * d + c] for t in range(len(keys))) for c in range(d)])
        out.append(ob)
    return out
