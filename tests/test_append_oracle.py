"""Pins of the append-path oracle: window ring and eviction against a plain token list."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import append as AP


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), W=st.integers(0, 6), n=st.integers(0, 25))
def test_ring_matches_token_list(seed, W, n):
    """After n appends to an empty sequence: latent rows are tokens 0..n-W'-1 projected in order
    (W' = min(W, n)), and the window holds the newest W' tokens, token p in slot p mod W."""
    rng = np.random.default_rng(seed)
    D, r = 6, 3
    P = rng.standard_normal((D, r))
    toks_k = rng.standard_normal((n, D))
    toks_v = rng.standard_normal((n, D))
    st_ = AP.SeqState(window=W, D=D)
    for i in range(n):
        AP.append_token(st_, toks_k[i], toks_v[i], P, P)
    Wn = min(W, n)
    assert st_.lat_len == n - Wn and st_.win_len == (Wn if W else 0)
    for t in range(n - Wn):
        assert st_.lat_pos[t] == t
        assert np.allclose(st_.lat_z_k[t], toks_k[t] @ P, rtol=0, atol=0)
        assert np.allclose(st_.lat_z_v[t], toks_v[t] @ P, rtol=0, atol=0)
    for p in range(n - Wn, n):
        assert np.array_equal(st_.ring_k[p % W], toks_k[p])
        assert np.array_equal(st_.ring_v[p % W], toks_v[p])


def test_identity_projection_is_exact():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(512)
    st_ = AP.SeqState(window=0, D=512)
    AP.append_token(st_, x, x, np.eye(512), np.eye(512))
    assert np.array_equal(st_.lat_z_k[0], x)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(10000) * 10.0 ** rng.integers(-5, 5, 10000)).astype(np.float32)
    x[:4] = [0.0, -0.0, np.inf, -np.inf]
    ours = AP.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
