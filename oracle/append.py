"""The append path: exact recent window, eviction into the latent history, projection, storage.

TEST INFRASTRUCTURE ONLY (see the package header).

iS-KV abstract: a recent window of tokens is kept exact while older states are
folded into the bounded-rank latent representation. TraceKV abstract: the cache
stores low-dimensional latents, optionally quantised. The workload projects a
new dense K/V row onto the latent space with the pseudo-inverse of the stored
basis, P = pinv(B) [D, r], supplied by the caller.

State of one sequence: L latent rows (positions 0..L-1) and W_b <= W window
tokens at positions L..L+W_b-1, each in ring slot (position mod W). Appending a
token x, one at a time, in arrival order:

  W == 0           z = x @ P is stored as latent row L; L += 1.
  W_b < W          x goes to slot (L + W_b) mod W; W_b += 1.
  W_b == W         the oldest window token (position L, slot L mod W, which is the
                   slot the new token takes) is projected, z = x_old @ P, and stored
                   as latent row L; L += 1; then x goes into that slot.

Storage of z: float32 caches keep f32(z); bf16 caches keep bf16_rne(f32(z));
int4 caches keep the Q1-Q5 quantisation of f32(z) (``oracle.quant``). z itself
is computed in float64 here.

Pins (tests/test_append_oracle.py): a brute-force list model of the token
stream (the latent rows are the oldest tokens in order, the window holds the
newest W in their slots) for random stream lengths; z = x exactly when P = I.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import quant


@dataclass
class SeqState:
    """One sequence of one layer, with dense window rows and float64 pre-storage z rows."""
    window: int
    D: int
    lat_z_k: list = field(default_factory=list)   # float64 [rank_k] per latent row
    lat_z_v: list = field(default_factory=list)
    lat_pos: list = field(default_factory=list)   # absolute position of each latent row
    ring_k: np.ndarray = None                     # [W, D] float64 (values as stored)
    ring_v: np.ndarray = None
    win_len: int = 0

    def __post_init__(self):
        if self.ring_k is None:
            self.ring_k = np.zeros((self.window, self.D))
            self.ring_v = np.zeros((self.window, self.D))

    @property
    def lat_len(self) -> int:
        return len(self.lat_z_k)


def append_token(st: SeqState, xk, xv, pk, pv, pos_base: int = 0) -> None:
    """Append one token (dense rows xk, xv [D]) following the rules in the module header.

    ``pos_base`` is the number of latent rows that existed before this state was
    created (positions are absolute)."""
    xk = np.asarray(xk, np.float64)
    xv = np.asarray(xv, np.float64)
    L = pos_base + st.lat_len
    if st.window == 0:
        st.lat_z_k.append(xk @ pk)
        st.lat_z_v.append(xv @ pv)
        st.lat_pos.append(L)
        return
    if st.win_len < st.window:
        slot = (L + st.win_len) % st.window
        st.ring_k[slot] = xk
        st.ring_v[slot] = xv
        st.win_len += 1
        return
    slot = L % st.window
    st.lat_z_k.append(st.ring_k[slot] @ pk)
    st.lat_z_v.append(st.ring_v[slot] @ pv)
    st.lat_pos.append(L)
    st.ring_k[slot] = xk
    st.ring_v[slot] = xv


def store_rows(z64: np.ndarray, latent: str):
    """Storage form of float64 rows z [n, r]: f32 array, bf16-valued f32 array, or int4 triple."""
    z32 = np.asarray(z64, np.float64).astype(np.float32)
    if latent == "f32":
        return z32
    if latent == "bf16":
        return bf16_rne(z32)
    if latent == "i4g32":
        return quant.quantize_rows(z32)
    raise ValueError(latent)


def bf16_rne(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.asarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(np.asarray(x32, np.float32))
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    out = np.where(nan, np.float32(np.nan), out)
    return out
