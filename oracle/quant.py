"""int4 group quantisation of latent rows (groups of 32 along the rank), float32 steps.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages fix only "4-bit quantization" on top of the low-rank latents (TraceKV
abstract; ai4snews page, Synopsis: 70% rank ratio with 4-bit quantisation).
The format below is the plainest reading of the stated workload: int4 codes in
groups of 32 consecutive latent indices, one float16 scale and one float16
zero per group, found by min-max over the group. Every step is one IEEE
operation in the precision written, so numpy float32/float16 reproduce it
exactly:

  Q1 groups     per row, indices [32 g, min(32 g + 32, r)); the last group may be
                partial and its min/max run over its real elements only.
  Q2 scale/zero zero16  = f16_rne(min)
                scale16 = f16_rne( f32( f32(max - min) / 15.0f ) )
  Q3 encode     code = clamp( rint_half_even( f32( f32(z - f32(zero16)) / f32(scale16) ) ), 0, 15 )
  Q4 degenerate scale16 == 0  ->  every code of the group is 0
  Q5 packing    16 bytes per group, two codes per byte, the even index in the low
                nibble; unused nibbles of a partial group are 0
  Q6 dequant    zhat = f32_rne( code * scale16 + zero16 ), one rounding. The exact
                value needs at most 45 significant bits (float16 values are
                multiples of 2**-24 below 2**16), so float64 holds it exactly and a
                single cast to float32 gives the correctly rounded result (the
                same as a fused multiply-add in float32).

Pins (tests/test_quant.py): exact-grid groups give codes k and zhat equal to the
input bitwise; degenerate and partial groups; nibble order; Q6 checked against
exact rational arithmetic; idempotence; error within scale/2 plus the float16
rounding of scale and zero.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
GROUP_BYTES = 16


def n_groups(rank: int) -> int:
    return (rank + GROUP - 1) // GROUP


def row_bytes(rank: int) -> int:
    """Packed code bytes per latent row."""
    return n_groups(rank) * GROUP_BYTES


def quantize_rows(z) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q1-Q5 on float32 rows z [n, r] -> (codes uint8 [n, G*16], scale f16 [n, G], zero f16 [n, G])."""
    z = np.asarray(z, dtype=np.float32)
    n, r = z.shape
    G = n_groups(r)
    codes = np.zeros((n, G * GROUP_BYTES), dtype=np.uint8)
    scale = np.zeros((n, G), dtype=np.float16)
    zero = np.zeros((n, G), dtype=np.float16)
    with np.errstate(all="ignore"):
        for g in range(G):
            lo, hi = g * GROUP, min(g * GROUP + GROUP, r)
            zg = z[:, lo:hi]
            mn = zg.min(axis=1)
            mx = zg.max(axis=1)
            z16 = mn.astype(np.float16)
            s16 = ((mx - mn) / np.float32(15.0)).astype(np.float16)
            z32 = z16.astype(np.float32)
            s32 = s16.astype(np.float32)
            c = np.rint((zg - z32[:, None]) / s32[:, None])
            c = np.clip(c, 0, 15)
            c[s16 == 0] = 0
            c = c.astype(np.uint8)
            scale[:, g] = s16
            zero[:, g] = z16
            for k in range(hi - lo):
                byte = g * GROUP_BYTES + k // 2
                if k % 2 == 0:
                    codes[:, byte] |= c[:, k]
                else:
                    codes[:, byte] |= (c[:, k] << 4).astype(np.uint8)
    return codes, scale, zero


def unpack_codes(codes: np.ndarray, rank: int) -> np.ndarray:
    """Q5 inverse: packed bytes [n, G*16] -> integer codes [n, rank]."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.zeros((codes.shape[0], rank), dtype=np.int64)
    for i in range(rank):
        g, k = divmod(i, GROUP)
        byte = codes[:, g * GROUP_BYTES + k // 2]
        out[:, i] = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
    return out


def dequant_rows(codes, scale, zero, rank: int) -> np.ndarray:
    """Q6: float32 [n, rank] with zhat = f32_rne(code * scale + zero), exact before the cast."""
    c = unpack_codes(codes, rank).astype(np.float64)
    gi = np.arange(rank) // GROUP
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)[:, gi]
    zz = np.asarray(zero, dtype=np.float16).astype(np.float64)[:, gi]
    return (c * s + zz).astype(np.float32)


def error_bound(scale, zero, rank: int) -> np.ndarray:
    """Per element bound on |zhat - z| for z quantised by Q1-Q5: half a step, plus the
    float16 rounding of zero (<= half an ulp) and of scale (15 steps times its half ulp),
    plus float32 rounding slack."""
    gi = np.arange(rank) // GROUP
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)
    zz = np.asarray(zero, dtype=np.float16).astype(np.float64)
    ulp_s = np.spacing(np.abs(np.asarray(scale, np.float16))).astype(np.float64)
    ulp_z = np.spacing(np.abs(np.asarray(zero, np.float16))).astype(np.float64)
    b = 0.5 * s + 0.5 * ulp_z + 15 * 0.5 * ulp_s + 4 * np.spacing(np.float32(1)) * (np.abs(zz) + 16 * s)
    return b[:, gi]


def pack_scale_zero(scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """Interleave float16 (scale, zero) pairs -> uint32 [n, G] (scale in the low half)."""
    s = np.asarray(scale, np.float16).view(np.uint16).astype(np.uint32)
    zz = np.asarray(zero, np.float16).view(np.uint16).astype(np.uint32)
    return s | (zz << 16)
