"""Pins of the int4 groups-of-32 quantiser oracle (Q1-Q6)."""
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked_example.txt")


def load_golden():
    cases = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, z, s, zz, codes, deq = [p.strip() for p in line.split("|")]
            cases[name] = dict(z=np.array([float(x) for x in z.split()], np.float32),
                               scale=float(s), zero=float(zz),
                               codes=bytes(int(h, 16) for h in codes.split()),
                               deq=np.array([float(x) for x in deq.split()], np.float32))
    return cases


@pytest.mark.parametrize("name", ["A", "B"])
def test_worked_example(name):
    c = load_golden()[name]
    codes, scale, zero = Q.quantize_rows(c["z"][None, :])
    assert float(scale[0, 0]) == c["scale"]
    assert float(zero[0, 0]) == c["zero"]
    assert bytes(codes[0]) == c["codes"]
    deq = Q.dequant_rows(codes, scale, zero, len(c["z"]))
    assert np.array_equal(deq[0], c["deq"])


def test_exact_grid_groups_roundtrip_bitwise():
    """z = zero + k * 2**-e with every k in 0..15 present: codes are k and zhat == z bitwise."""
    rng = np.random.default_rng(0)
    n, r = 64, 358
    G = Q.n_groups(r)
    z = np.zeros((n, r), np.float32)
    k_all = np.zeros((n, r), np.int64)
    for i in range(n):
        for g in range(G):
            lo, hi = g * 32, min(g * 32 + 32, r)
            m = hi - lo
            k = rng.integers(0, 16, size=m)
            k[0], k[-1] = 0, 15
            rng.shuffle(k)
            e = int(rng.integers(2, 8))
            z0 = np.float16(rng.standard_normal()).astype(np.float64)
            z0 = np.round(z0 * 2 ** e) / 2 ** e        # on the grid, exact in float16
            z[i, lo:hi] = (z0 + k * 2.0 ** -e).astype(np.float32)
            k_all[i, lo:hi] = k
    codes, scale, zero = Q.quantize_rows(z)
    assert np.array_equal(Q.unpack_codes(codes, r), k_all)
    assert np.array_equal(Q.dequant_rows(codes, scale, zero, r).view(np.uint32), z.view(np.uint32))


def test_degenerate_group_codes_zero():
    z = np.full((3, 40), 0.7, np.float32)
    z[1, 32:] = -2.5      # second group degenerate at another value
    codes, scale, zero = Q.quantize_rows(z)
    assert np.all(Q.unpack_codes(codes, 40) == 0)
    assert np.all(scale == 0)
    deq = Q.dequant_rows(codes, scale, zero, 40)
    assert np.array_equal(deq, np.float16(z).astype(np.float32))


def test_partial_last_group_uses_real_elements_only():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 358)).astype(np.float32)
    c1, s1, z1 = Q.quantize_rows(z)
    wide = np.concatenate([z, np.full((5, 26), 1e4, np.float32)], axis=1)  # 384 = 12 full groups
    c2, s2, z2 = Q.quantize_rows(wide)
    assert np.array_equal(s1[:, :11], s2[:, :11]) and np.array_equal(c1[:, :176], c2[:, :176])
    assert not np.array_equal(s1[:, 11], s2[:, 11])
    # the partial group's unused nibbles are zero: 6 codes -> 3 bytes, then 13 zero bytes
    assert np.all(c1[:, 176 + 3:] == 0)
    assert c1.shape == (5, 12 * 16)


def test_nibble_order_even_low():
    z = np.zeros((1, 32), np.float32)
    z[0, :] = 0.0
    z[0, 1] = 15.0                       # scale 1, zero 0 -> code[1] = 15, others 0
    codes, scale, zero = Q.quantize_rows(z)
    assert float(scale[0, 0]) == 1.0
    assert codes[0, 0] == 0xF0 and np.all(codes[0, 1:] == 0)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), scale_exp=st.integers(-12, 6))
def test_dequant_is_single_rounding_of_exact_value(seed, scale_exp):
    """Q6 against exact rational arithmetic: f32_rne(code * scale + zero)."""
    rng = np.random.default_rng(seed)
    r = 64
    z = (rng.standard_normal((2, r)) * 2.0 ** scale_exp).astype(np.float32)
    codes, scale, zero = Q.quantize_rows(z)
    deq = Q.dequant_rows(codes, scale, zero, r)
    cc = Q.unpack_codes(codes, r)
    for i in range(2):
        for k in range(0, r, 7):
            g = k // 32
            exact = Fraction(int(cc[i, k])) * Fraction(float(scale[i, g])) + Fraction(float(zero[i, g]))
            f = float(exact)                     # correctly rounded to float64 (exact here)
            assert Fraction(f) == exact          # the value fits in float64
            assert np.float32(f) == deq[i, k]    # one rounding to float32


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), r=st.integers(1, 200), mag=st.integers(-6, 6))
def test_error_bound_and_idempotence(seed, r, mag):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((4, r)) * 2.0 ** mag).astype(np.float32)
    codes, scale, zero = Q.quantize_rows(z)
    deq = Q.dequant_rows(codes, scale, zero, r)
    assert np.all(np.abs(deq.astype(np.float64) - z) <= Q.error_bound(scale, zero, r))
    c2, s2, z2 = Q.quantize_rows(deq)
    d2 = Q.dequant_rows(c2, s2, z2, r)
    # re-quantising the dequantised values changes nothing beyond one float32 ulp
    assert np.all(np.abs(d2.astype(np.float64) - deq) <= 2 * np.spacing(np.abs(deq)) + 1e-30)


def test_codes_within_range_and_monotone():
    rng = np.random.default_rng(3)
    z = np.sort(rng.standard_normal((8, 32)).astype(np.float32), axis=1)
    codes, _, _ = Q.quantize_rows(z)
    c = Q.unpack_codes(codes, 32)
    assert c.min() == 0 and c.max() == 15
    assert np.all(np.diff(c, axis=1) >= 0)


def test_pack_scale_zero_layout():
    s = np.array([[1.0, 0.5]], np.float16)
    zz = np.array([[-2.0, 0.25]], np.float16)
    w = Q.pack_scale_zero(s, zz)
    assert w[0, 0] == (0x3C00 | (0xC000 << 16))
    assert w[0, 1] == (0x3800 | (0x3400 << 16))
