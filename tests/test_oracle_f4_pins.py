"""Pins of the oracle's cross-attention and of the naive-patch variant.

Cross-attention (patch queries over a context every patch shares) is pinned
against torch's fp64 scaled_dot_product_attention, brute force on tiny
inputs, and the closed forms of uniform and single-token contexts.

The naive-patch baseline (each patch alone, no context from the others: the
README mirror's figure (b)) is the oracle's layers at n = 1 on the patch's
rows.  It is pinned against torch's library layers on the patch alone, and
against the property the pages give it: seams.  With stale = fresh the
displaced layer reproduces the full-image rows exactly, while the naive conv
differs from them in the patch's first and last rows only, and the naive
attention and GroupNorm differ everywhere.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic_inputs as si


def _ctx(B=2, Lq=37, Lk=77, heads=3, d=64, seed=7):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, Lq, heads, d)), g.standard_normal((B, Lk, heads, d)),
            g.standard_normal((B, Lk, heads, d)))


def test_cross_attention_matches_sdpa():
    q, k, v = _ctx()
    out = oracle.cross_attn(0.125, q, k, v)
    t = lambda a: torch.from_numpy(a).transpose(1, 2)
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.125).transpose(1, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_cross_attention_brute_force():
    q, k, v = _ctx(B=1, Lq=3, Lk=5, heads=2, d=4, seed=3)
    out = oracle.cross_attn(0.7, q, k, v)
    for b in range(1):
        for r in range(3):
            for hd in range(2):
                s = [0.7 * sum(q[b, r, hd, e] * k[b, t, hd, e] for e in range(4)) for t in range(5)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                for e in range(4):
                    ref = sum(w[t] * v[b, t, hd, e] for t in range(5)) / z
                    assert abs(out[b, r, hd, e] - ref) < 1e-12


def test_cross_attention_closed_forms():
    q, k, v = _ctx(Lk=9)
    k_same = np.broadcast_to(k[:, :1], k.shape).copy()   # identical keys: mean of V
    np.testing.assert_allclose(oracle.cross_attn(0.125, q, k_same, v), np.broadcast_to(
        v.mean(axis=1, keepdims=True), q.shape), rtol=1e-12, atol=1e-13)
    one = oracle.cross_attn(0.125, q, k[:, :1], v[:, :1])  # one token: its V
    np.testing.assert_allclose(one, np.broadcast_to(v[:, :1], q.shape), rtol=0, atol=1e-15)


def _naive(geom):
    B, H, W, n, i = geom
    return (B, H // n, W, 1, 0)


def _libs_on_patch(wl, d):
    """torch library layers applied to the patch rows alone."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    x = t(d["x_fresh"].double().numpy()).permute(0, 3, 1, 2)
    conv = F.conv2d(x, t(d["weight"].double().numpy()).permute(0, 3, 1, 2), t(d["bias"].double().numpy()),
                    padding=1).permute(0, 2, 3, 1).numpy()
    gn = F.group_norm(x, wl.groups, t(d["gamma"].double().numpy()), t(d["beta"].double().numpy()),
                      wl.eps).permute(0, 2, 3, 1).numpy()
    qt = lambda a: t(a.double().numpy()).transpose(1, 2)
    att = F.scaled_dot_product_attention(qt(d["q"]), qt(d["k_fresh"]), qt(d["v_fresh"]),
                                         scale=wl.head_dim ** -0.5).transpose(1, 2).numpy()
    return conv, gn, att


@pytest.mark.parametrize("patch", [0, 1])
def test_naive_patch_is_the_layer_on_the_patch_alone(patch):
    wl = si.WORKLOADS["tiny"].with_patch(patch)
    d = si.make_inputs(wl, nonzero_bias=True)
    ng = _naive(wl.geom)
    conv = oracle.patch_conv3x3_halo(ng, wl.channels, wl.channels, d["x_fresh"], None, d["weight"],
                                     d["bias"])
    gn, _ = oracle.async_groupnorm(ng, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                   np.zeros((wl.batch, 1, wl.groups, 2)), d["gamma"], d["beta"])
    att = oracle.patch_self_attn(ng, wl.heads, wl.head_dim, wl.head_dim ** -0.5, d["q"], d["k_fresh"],
                                 d["v_fresh"], None, None)
    rc, rg, ra = _libs_on_patch(wl, d)
    np.testing.assert_allclose(conv, rc, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(gn, rg, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(att, ra, rtol=1e-10, atol=1e-12)


def test_naive_patch_has_seams_displaced_has_none():
    wl = si.WORKLOADS["tiny"].with_patch(1)
    d = si.make_inputs(wl, stale_equals_fresh=True, nonzero_bias=True)
    B, H, W, C, h, i = wl.batch, wl.height, wl.width, wl.channels, wl.h, wl.patch
    full = (B, H, W, 1, 0)
    xs = d["x_stale"]                                    # = the full current map
    full_conv = oracle.patch_conv3x3_halo(full, C, C, xs, None, d["weight"], d["bias"])[:, i * h:(i + 1) * h]
    disp = oracle.patch_conv3x3_halo(wl.geom, C, C, d["x_fresh"], xs, d["weight"], d["bias"])
    naive = oracle.patch_conv3x3_halo(_naive(wl.geom), C, C, d["x_fresh"], None, d["weight"], d["bias"])
    np.testing.assert_allclose(disp, full_conv, rtol=1e-12, atol=1e-12)
    diff = np.abs(naive - full_conv).max(axis=(0, 2, 3))   # per local row
    assert diff[0] > 1e-3                                  # the row next to patch 0: a seam
    assert np.all(diff[1:h - 1] < 1e-12)                   # interior rows agree
    # patch 1 of 2 is the bottom patch: its last row is the image edge, no seam
    assert diff[h - 1] < 1e-12
    # attention and GroupNorm see only the patch: they differ everywhere
    Lq = wl.lq
    att_full = oracle.patch_self_attn(wl.geom, wl.heads, 64, 0.125, d["q"], d["k_fresh"], d["v_fresh"],
                                      d["k_stale"], d["v_stale"])
    att_naive = oracle.patch_self_attn(_naive(wl.geom), wl.heads, 64, 0.125, d["q"], d["k_fresh"],
                                       d["v_fresh"], None, None)
    assert np.abs(att_full - att_naive).max(axis=(0, 2, 3)).min() > 1e-6
    assert att_full.shape == (B, Lq, wl.heads, 64)
