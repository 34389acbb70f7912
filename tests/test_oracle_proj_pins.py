"""Pins of the oracle's projection functions (CPU).

oracle.linear and oracle.patch_qkv_proj are checked against things other
than themselves: numpy's matmul (a library routine), pure-Python loops on
tiny inputs, the closed form of an identity weight, and the refresh rule
(patch rows replaced, all other rows untouched)."""
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("M,C,N", [(1, 1, 1), (7, 5, 3), (64, 48, 96), (33, 64, 192)])
def test_linear_matches_numpy_matmul(M, C, N):
    r = _rng(M * 1000 + C * 10 + N)
    x = r.standard_normal((M, C))
    w = r.standard_normal((N, C))
    b = r.standard_normal(N)
    np.testing.assert_allclose(oracle.linear(x, w, b), x @ w.T + b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.linear(x, w), x @ w.T, rtol=1e-12, atol=1e-12)


def test_linear_brute_force_tiny():
    r = _rng(3)
    x = r.standard_normal((2, 3, 4))
    w = r.standard_normal((5, 4))
    b = r.standard_normal(5)
    y = oracle.linear(x, w, b)
    for i in range(2):
        for j in range(3):
            for o in range(5):
                acc = b[o]
                for c in range(4):
                    acc += w[o, c] * x[i, j, c]
                assert math.isclose(y[i, j, o], acc, rel_tol=1e-13, abs_tol=1e-13)


def test_identity_weight_gives_input_plus_bias():
    r = _rng(4)
    x = r.standard_normal((3, 10, 16))
    b = r.standard_normal(16)
    np.testing.assert_array_equal(oracle.linear(x, np.eye(16), b), x + b)


@pytest.mark.parametrize("patch", [0, 2, 3])
def test_qkv_split_and_fused_refresh(patch):
    B, H, W, n, C = 2, 8, 3, 4, 6
    geom = (B, H, W, n, patch)
    h = H // n
    Lq = h * W
    r = _rng(10 + patch)
    x = r.standard_normal((B, h, W, C))
    w = r.standard_normal((3 * C, C))
    b = r.standard_normal(3 * C)
    ks = r.standard_normal((B, H * W, C))
    vs = r.standard_normal((B, H * W, C))
    q, k, v, ks2, vs2 = oracle.patch_qkv_proj(geom, C, x, w, b, ks, vs)
    full = x.reshape(B, Lq, C) @ w.T + b
    np.testing.assert_allclose(q, full[..., :C], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k, full[..., C:2 * C], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v, full[..., 2 * C:], rtol=1e-12, atol=1e-12)
    lo, hi = patch * Lq, (patch + 1) * Lq
    np.testing.assert_array_equal(ks2[:, lo:hi], k)
    np.testing.assert_array_equal(vs2[:, lo:hi], v)
    outside = np.ones(H * W, dtype=bool)
    outside[lo:hi] = False
    np.testing.assert_array_equal(ks2[:, outside], ks[:, outside])
    np.testing.assert_array_equal(vs2[:, outside], vs[:, outside])
    # inputs are not modified
    assert not np.shares_memory(ks2, ks)


def test_qkv_without_stale_maps():
    geom = (1, 4, 2, 2, 1)
    r = _rng(20)
    x = r.standard_normal((1, 2, 2, 4))
    w = r.standard_normal((12, 4))
    q, k, v, ks, vs = oracle.patch_qkv_proj(geom, 4, x, w)
    assert ks is None and vs is None
    np.testing.assert_allclose(np.concatenate([q, k, v], -1), x.reshape(1, 4, 4) @ w.T, rtol=1e-12)


def test_qkv_rejects_bad_geometry():
    with pytest.raises(ValueError):
        oracle.patch_qkv_proj((1, 5, 2, 2, 0), 4, np.zeros((1, 2, 2, 4)), np.zeros((12, 4)))
