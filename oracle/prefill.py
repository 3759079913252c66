"""Chunked prefill attention over a low-rank latent KV cache: plain float64 definitions.

TEST INFRASTRUCTURE ONLY (see the package header).

TraceKV (abstract): the cache keeps low-dimensional latents of the KV states of "large
multimodal contexts" and growing reasoning traces; attention runs from those latents. The pages
describe decode; prefill of a prompt chunk over an existing latent history is not spelled out.
The plainest reading, used here: a chunk of C new tokens of sequence b arrives with exact
(dense) keys and values k_new, v_new [C, D]. Query token c attends, causally, to

    the latent history      K = Zk[:L] Bk,  V = Zv[:L] Bv        (positions 0 .. L-1)
    the exact window ring   win_len[b] rows at positions L .. L+win_len-1
    the chunk itself        k_new[0 .. c], v_new[0 .. c]

with head j using KV head g = j // (Hq / Hkv), scores sm_scale * q . K[:, g], softmax over that
union and the weighted sum of V[:, g]. Storing the chunk afterwards (projection, quantisation,
window eviction) is the append path's job, not part of this function.

Functions
---------
``prefill_reconstruct``  P1: reconstruct K and V, then causal softmax attention (primary).
``prefill_latent``       P2: the latent-domain computation: fold each query into the latent
                         space, score latent keys there, accumulate latent values, up-project
                         once; the window and chunk keys are scored exactly.
``prefill_bruteforce``   P3: P1 with Python loops (tiny shapes).

Pins (tests/test_prefill_oracle.py): P1 = P2 to 1e-12; full rank with identity bases equals
torch's scaled_dot_product_attention under an explicit mask that aligns the chunk's queries
with the end of the key sequence; a one-token chunk equals the decode oracle with that token
appended to the exact window; causality (later chunk tokens do not change earlier outputs);
the first chunk token of an empty cache returns its own value; P3 on random tiny shapes.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .attention import _f64, _softmax, window_rows


def _exact_rows(b, L, kwin, vwin, win_len, window, D):
    if window and win_len is not None and int(win_len[b]) > 0:
        wl = int(win_len[b])
        return window_rows(_f64(kwin[b]), L, wl, window), window_rows(_f64(vwin[b]), L, wl, window)
    return np.zeros((0, D)), np.zeros((0, D))


def prefill_reconstruct(q, zk, zv, bk, bv, lat_len: Sequence[int], rank_k: int, rank_v: int,
                        n_kv_heads: int, sm_scale: float, k_new, v_new, kwin=None, vwin=None,
                        win_len: Optional[Sequence[int]] = None, window: int = 0,
                        batches: Optional[Sequence[int]] = None) -> np.ndarray:
    """P1. q [B, C, Hq, d]; k_new, v_new [B, C, D]; latents and rings as for decode.
    Returns float64 [len(batches), C, Hq, d]."""
    q = _f64(q)
    bk = _f64(bk)[:rank_k]
    bv = _f64(bv)[:rank_v]
    k_new = _f64(k_new)
    v_new = _f64(v_new)
    B, C, Hq, d = q.shape
    D = bk.shape[1]
    grp = Hq // n_kv_heads
    batches = range(B) if batches is None else batches
    out = np.zeros((len(batches), C, Hq, d))
    for i, b in enumerate(batches):
        L = int(lat_len[b])
        Kw, Vw = _exact_rows(b, L, kwin, vwin, win_len, window, D)
        K = np.concatenate([_f64(zk[b][:L])[:, :rank_k] @ bk, Kw, k_new[b]], axis=0)
        V = np.concatenate([_f64(zv[b][:L])[:, :rank_v] @ bv, Vw, v_new[b]], axis=0)
        n0 = L + Kw.shape[0]                       # keys before the chunk
        for c in range(C):
            n = n0 + c + 1
            for g in range(n_kv_heads):
                heads = slice(g * grp, (g + 1) * grp)
                cols = slice(g * d, (g + 1) * d)
                s = sm_scale * (K[:n, cols] @ q[b, c, heads].T)     # [n, grp]
                out[i, c, heads] = _softmax(s, axis=0).T @ V[:n, cols]
    return out


def prefill_latent(q, zk, zv, bk, bv, lat_len: Sequence[int], rank_k: int, rank_v: int,
                   n_kv_heads: int, sm_scale: float, k_new, v_new, kwin=None, vwin=None,
                   win_len: Optional[Sequence[int]] = None, window: int = 0,
                   batches: Optional[Sequence[int]] = None) -> np.ndarray:
    """P2, the steps in the library's order:

    1. fold:       qt_{c,j} = q_{c,j} @ Bk[:, g]^T                         [rank_k]
    2. scores:     latent  s_t = sm_scale * Zk[t] . qt_{c,j}
                   exact   s_e = sm_scale * q_{c,j} . K_e[g]  (window rows, chunk rows <= c)
    3. softmax over the union
    4. accumulate: A_{c,j} = sum_t p_t Zv[t]                               [rank_v]
    5. up-project: o_{c,j} = A_{c,j} @ Bv[:, g] + sum_e p_e V_e[g]
    """
    q = _f64(q)
    bk = _f64(bk)[:rank_k]
    bv = _f64(bv)[:rank_v]
    k_new = _f64(k_new)
    v_new = _f64(v_new)
    B, C, Hq, d = q.shape
    D = bk.shape[1]
    grp = Hq // n_kv_heads
    batches = range(B) if batches is None else batches
    out = np.zeros((len(batches), C, Hq, d))
    for i, b in enumerate(batches):
        L = int(lat_len[b])
        Zk = _f64(zk[b][:L])[:, :rank_k]
        Zv = _f64(zv[b][:L])[:, :rank_v]
        Kw, Vw = _exact_rows(b, L, kwin, vwin, win_len, window, D)
        for c in range(C):
            Ke = np.concatenate([Kw, k_new[b, :c + 1]], axis=0)
            Ve = np.concatenate([Vw, v_new[b, :c + 1]], axis=0)
            for g in range(n_kv_heads):
                heads = slice(g * grp, (g + 1) * grp)
                cols = slice(g * d, (g + 1) * d)
                qc = q[b, c, heads]                              # [grp, d]
                qt = qc @ bk[:, cols].T                          # [grp, rank_k]
                s_lat = sm_scale * (Zk @ qt.T)                    # [L, grp]
                s_ex = sm_scale * (Ke[:, cols] @ qc.T)            # [E, grp]
                p = _softmax(np.concatenate([s_lat, s_ex], axis=0), axis=0)
                A = p[:L].T @ Zv                                  # [grp, rank_v]
                out[i, c, heads] = A @ bv[:, cols] + p[L:].T @ Ve[:, cols]
    return out


def prefill_bruteforce(q, zk, zv, bk, bv, lat_len, rank_k, rank_v, n_kv_heads, sm_scale,
                       k_new, v_new):
    """P3: P1 without a window, nested Python loops and math.exp only (tiny shapes)."""
    B, C, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    D = len(bk[0])
    grp = Hq // n_kv_heads
    out = []
    for b in range(B):
        L = int(lat_len[b])
        keys, vals = [], []
        for t in range(L):
            keys.append([sum(float(zk[b][t][i]) * float(bk[i][x]) for i in range(rank_k)) for x in range(D)])
            vals.append([sum(float(zv[b][t][i]) * float(bv[i][x]) for i in range(rank_v)) for x in range(D)])
        ob = []
        for c in range(C):
            ks = keys + [[float(x) for x in k_new[b][e]] for e in range(c + 1)]
            vs = vals + [[float(x) for x in v_new[b][e]] for e in range(c + 1)]
            oc = []
            for j in range(Hq):
                g = j // grp
                s = [sm_scale * sum(float(q[b][c][j][x]) * k[g * d + x] for x in range(d)) for k in ks]
                m = max(s)
                e = [math.exp(v - m) for v in s]
                tot = sum(e)
                oc.append([sum(e[t] / tot * vs[t][g * d + x] for t in range(len(ks))) for x in range(d)])
            ob.append(oc)
        out.append(ob)
    return out
