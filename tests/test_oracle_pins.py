"""Pins of the CPU oracle against things other than itself (CPU only).

* hand-derived worked examples (tests/golden/hand_examples.json);
* the hybrid-map identity: the patch layer equals torch's float64 library
  layer (SDPA, conv2d, group_norm) on the hybrid map, restricted to the
  patch's rows, on every workload shape;
* stale == fresh gives the full-image layer; n == 1 gives the full layer with
  the stale inputs never read;
* brute force in pure Python on tiny inputs;
* closed forms (constant keys, a single token, the variance clamp, conv
  linearity) and NaN-poison invariants for the parts the method must not read.
"""
import functools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tests import brute, libref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _arr(x):
    return np.array(x, dtype=np.float64)


@functools.lru_cache(maxsize=4)
def _inputs(name, patch, stale_equals_fresh=False, nonzero_bias=True):
    wl = si.WORKLOADS[name].with_patch(patch)
    return wl, si.make_inputs(wl, stale_equals_fresh=stale_equals_fresh, nonzero_bias=nonzero_bias)


def _relmax(a, b):
    b = np.asarray(b)
    return float(np.max(np.abs(np.asarray(a) - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


# --------------------------------------------------------------------------- golden
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_attention_two_tokens():
    g = _golden()["attention_two_tokens"]
    out = oracle.patch_self_attn(tuple(g["geom"]), g["heads"], g["head_dim"], g["scale"],
                                 _arr(g["q"]), _arr(g["k_fresh"]), _arr(g["v_fresh"]),
                                 _arr(g["k_stale"]), _arr(g["v_stale"]))
    np.testing.assert_allclose(out, _arr(g["expected"]), rtol=0, atol=1e-14)


def test_golden_conv_halo():
    g = _golden()["conv_halo_from_above"]
    y = oracle.patch_conv3x3_halo(tuple(g["geom"]), g["c_in"], g["c_out"], _arr(g["x_fresh"]),
                                  _arr(g["x_stale"]), _arr(g["weight"]), _arr(g["bias"]))
    np.testing.assert_allclose(y, _arr(g["expected"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("key", ["groupnorm_mixed_moments", "groupnorm_clamped_variance"])
def test_golden_groupnorm(key):
    g = _golden()[key]
    y, fm = oracle.async_groupnorm(tuple(g["geom"]), g["channels"], g["groups"], g["eps"],
                                   _arr(g["x_fresh"]), _arr(g["stale_moments"]))
    np.testing.assert_allclose(y, _arr(g["expected"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fm, _arr(g["expected_fresh_moments"]), rtol=0, atol=1e-14)


def test_golden_refresh():
    g = _golden()["refresh_rows"]
    s = oracle.refresh_stale(tuple(g["geom"]), g["row_elems"], _arr(g["fresh"]), _arr(g["stale"]))
    np.testing.assert_array_equal(s, _arr(g["expected"]))


# --------------------------------------------------------------- library pins
ALL_PATCH = [("tiny", 0), ("tiny", 1)]
SAMPLED = [("sdxl1024_l2", 0), ("sdxl1024_l2", 4), ("sdxl1024_l2", 7), ("sdxl1024_l3", 1),
           ("sdxl1024_l3", 3), ("sdxl2048_l2", 4), ("sdxl3840_l2", 4), ("sdxl3840_l3", 7)]


def _sample_rows(wl, count):
    """A few local query rows: first, last and a middle band."""
    if wl.lq <= count:
        return (0, wl.lq)
    mid = wl.lq // 2
    return (mid, mid + count)


@pytest.mark.parametrize("name,patch", ALL_PATCH + SAMPLED)
def test_attention_matches_sdpa_on_hybrid_map(name, patch):
    wl, d = _inputs(name, patch)
    rows = (0, wl.lq) if name == "tiny" else _sample_rows(wl, 4 if wl.tokens > 20000 else 16)
    scale = 1.0 / math.sqrt(wl.head_dim)
    args = (d["q"], d["k_fresh"], d["v_fresh"], d["k_stale"], d["v_stale"])
    got = oracle.patch_self_attn(wl.geom, wl.heads, wl.head_dim, scale, *args, rows=rows)
    ref = libref.attn_ref(wl.geom, scale, *args, rows=rows)
    assert _relmax(got, ref) < 1e-12


@pytest.mark.parametrize("name,patch", ALL_PATCH + SAMPLED)
def test_conv_matches_conv2d_on_hybrid_map(name, patch):
    wl, d = _inputs(name, patch)
    h = wl.h
    # first and last local rows carry the halo; one interior row besides
    row_sets = [(0, h)] if name == "tiny" else [(0, 1), (h - 1, h)]
    for rows in row_sets:
        got = oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, d["x_fresh"],
                                        d["x_stale"], d["weight"], d["bias"], rows=rows)
        ref = libref.conv_ref(wl.geom, d["x_fresh"], d["x_stale"], d["weight"], d["bias"], rows=rows)
        assert _relmax(got, ref) < 1e-12, rows


@pytest.mark.parametrize("name,patch", ALL_PATCH + SAMPLED)
def test_groupnorm_matches_group_norm_on_hybrid_map(name, patch):
    wl, d = _inputs(name, patch)
    # the previous step's per-patch moments of the stale map (numpy means)
    table = libref.patch_moments(d["x_stale"], wl.geom, wl.groups)
    y, fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"], table,
                                   d["gamma"], d["beta"])
    ref = libref.gn_ref(wl.geom, wl.groups, wl.eps, d["x_fresh"], d["x_stale"], d["gamma"], d["beta"])
    assert _relmax(y, ref) < 1e-10
    # fresh moments are those of the fresh slice (patch 0 of a 1-patch map)
    xf = d["x_fresh"]
    own = libref.patch_moments(xf, (wl.batch, xf.shape[1], wl.width, 1, 0), wl.groups)[:, 0]
    np.testing.assert_allclose(fm, own, rtol=1e-12, atol=1e-14)


# ------------------------------------------------- special cases of the method
def test_stale_equals_fresh_gives_full_image_layer():
    """With stale == fresh the hybrid map is the full map: the patch layer must
    equal the full-image layer's rows for that patch."""
    for patch in (0, 1):
        wl, d = _inputs("tiny", patch, stale_equals_fresh=True)
        full = {k: v for k, v in d.items()}
        scale = 0.125
        got = oracle.patch_self_attn(wl.geom, wl.heads, 64, scale, d["q"], d["k_fresh"], d["v_fresh"],
                                     d["k_stale"], d["v_stale"])
        # full-image layer: every token from the (unperturbed) full map
        ref = torch.nn.functional.scaled_dot_product_attention(
            d["q"].double().permute(0, 2, 1, 3), full["k_stale"].double().permute(0, 2, 1, 3),
            full["v_stale"].double().permute(0, 2, 1, 3), scale=scale).permute(0, 2, 1, 3).numpy()
        assert _relmax(got, ref) < 1e-12
        y = oracle.patch_conv3x3_halo(wl.geom, 128, 128, d["x_fresh"], d["x_stale"], d["weight"], d["bias"])
        xs = d["x_stale"].double().permute(0, 3, 1, 2)
        yr = torch.nn.functional.conv2d(xs, d["weight"].double().permute(0, 3, 1, 2), d["bias"].double(),
                                        padding=1)[:, :, patch * 16:(patch + 1) * 16]
        assert _relmax(y, yr.permute(0, 2, 3, 1).numpy()) < 1e-12
        table = libref.patch_moments(d["x_stale"], wl.geom, wl.groups)
        g, _ = oracle.async_groupnorm(wl.geom, 128, 32, 1e-5, d["x_fresh"], table, d["gamma"], d["beta"])
        gr = torch.nn.functional.group_norm(xs, 32, d["gamma"].double(), d["beta"].double(), 1e-5)
        gr = gr[:, :, patch * 16:(patch + 1) * 16].permute(0, 2, 3, 1).numpy()
        assert _relmax(g, gr) < 1e-10


def test_one_patch_is_the_full_layer_and_reads_no_stale():
    wl = si.Workload("one", 2, 16, 6, 5, 1, 2, head_dim=8, groups=4, dtype="f32", seed=77)
    d = si.make_inputs(wl, nonzero_bias=True)
    nan_tok = np.full(d["k_stale"].shape, np.nan)
    nan_map = np.full(d["x_stale"].shape, np.nan)
    got = oracle.patch_self_attn(wl.geom, 2, 8, 0.3, d["q"], d["k_fresh"], d["v_fresh"], nan_tok, nan_tok)
    ref = torch.nn.functional.scaled_dot_product_attention(
        d["q"].double().permute(0, 2, 1, 3), d["k_fresh"].double().permute(0, 2, 1, 3),
        d["v_fresh"].double().permute(0, 2, 1, 3), scale=0.3).permute(0, 2, 1, 3).numpy()
    assert _relmax(got, ref) < 1e-12
    y = oracle.patch_conv3x3_halo(wl.geom, 16, 16, d["x_fresh"], nan_map, d["weight"], d["bias"])
    xf = d["x_fresh"].double().permute(0, 3, 1, 2)
    yr = torch.nn.functional.conv2d(xf, d["weight"].double().permute(0, 3, 1, 2), d["bias"].double(), padding=1)
    assert _relmax(y, yr.permute(0, 2, 3, 1).numpy()) < 1e-12
    g, _ = oracle.async_groupnorm(wl.geom, 16, 4, 1e-5, d["x_fresh"], np.full((2, 1, 4, 2), np.nan),
                                  d["gamma"], d["beta"])
    gr = torch.nn.functional.group_norm(xf, 4, d["gamma"].double(), d["beta"].double(), 1e-5)
    assert _relmax(g, gr.permute(0, 2, 3, 1).numpy()) < 1e-10


TINY_GEOMS = [(1, 4, 4, 1, 0), (2, 4, 3, 2, 0), (1, 4, 5, 2, 1), (1, 8, 4, 4, 0), (2, 8, 3, 4, 2),
              (1, 8, 4, 4, 3)]


@pytest.mark.parametrize("geom", TINY_GEOMS)
def test_brute_force_tiny(geom):
    B, H, W, n, i = geom
    rng = np.random.default_rng(sum(geom) * 31 + i)
    h, L = H // n, H * W
    Lq = h * W
    heads, d = 2, 4
    q = rng.standard_normal((B, Lq, heads, d))
    kf, vf = rng.standard_normal((B, Lq, heads, d)), rng.standard_normal((B, Lq, heads, d))
    ks, vs = rng.standard_normal((B, L, heads, d)), rng.standard_normal((B, L, heads, d))
    got = oracle.patch_self_attn(geom, heads, d, 0.7, q, kf, vf, ks, vs)
    assert _relmax(got, np.array(brute.attention(geom, 0.7, q, kf, vf, ks, vs))) < 1e-12

    C, Co, G = 8, 6, 2
    xf, xs = rng.standard_normal((B, h, W, C)), rng.standard_normal((B, H, W, C))
    w, bias = rng.standard_normal((Co, 3, 3, C)), rng.standard_normal(Co)
    y = oracle.patch_conv3x3_halo(geom, C, Co, xf, xs, w, bias)
    assert _relmax(y, np.array(brute.conv3x3(geom, xf, xs, w, bias))) < 1e-12

    gamma, beta = rng.standard_normal(C), rng.standard_normal(C)
    table = libref.patch_moments(xs, geom, G)
    yg, _ = oracle.async_groupnorm(geom, C, G, 1e-5, xf, table, gamma, beta)
    assert _relmax(yg, np.array(brute.groupnorm(geom, G, 1e-5, xf, xs, gamma, beta))) < 1e-10


def test_constant_keys_give_mean_of_values():
    """Equal scores everywhere: the output is the plain mean of the hybrid V."""
    geom = (1, 4, 3, 2, 1)
    rng = np.random.default_rng(5)
    Lq, L = 6, 12
    q = rng.standard_normal((1, Lq, 1, 4))
    kf = np.tile(np.array([0.3, -1.0, 2.0, 0.5]), (1, Lq, 1, 1))
    ks = np.tile(np.array([0.3, -1.0, 2.0, 0.5]), (1, L, 1, 1))
    vf, vs = rng.standard_normal((1, Lq, 1, 4)), rng.standard_normal((1, L, 1, 4))
    out = oracle.patch_self_attn(geom, 1, 4, 1.0, q, kf, vf, ks, vs)
    mean_v = (vs[0, :6, 0].sum(0) + vf[0, :, 0].sum(0)) / L  # tokens 0..5 stale, 6..11 fresh
    np.testing.assert_allclose(out[0, :, 0], np.tile(mean_v, (Lq, 1)), rtol=1e-12, atol=1e-13)


def test_single_token_gives_its_value():
    q = np.array([[[[2.0, -1.0]]]])
    v = np.array([[[[0.25, 4.0]]]])
    out = oracle.patch_self_attn((1, 1, 1, 1, 0), 1, 2, 5.0, q, q, v, q * np.nan, v * np.nan)
    np.testing.assert_array_equal(out, v)


def test_forced_clamp_closed_form():
    geom = (1, 4, 2, 2, 0)
    rng = np.random.default_rng(9)
    xf = rng.standard_normal((1, 2, 2, 4))
    m = oracle.group_moments(xf, 1)
    table = np.zeros((1, 2, 1, 2))
    table[0, 0] = np.nan
    table[0, 1] = [10.0, 0.0]  # E[x^2] far below E[x]^2: mixed variance < 0
    gamma, beta = rng.standard_normal(4), rng.standard_normal(4)
    y, _ = oracle.async_groupnorm(geom, 4, 1, 1e-3, xf, table, gamma, beta)
    mu = (m[0, 0, 0] + 10.0) / 2
    assert (m[0, 0, 1] + 0.0) / 2 - mu * mu < 0
    np.testing.assert_allclose(y, (xf - mu) / math.sqrt(1e-3) * gamma + beta, rtol=1e-12)


def test_conv_is_linear_in_input_and_weight():
    geom = (1, 6, 4, 3, 1)
    rng = np.random.default_rng(3)
    xf1, xf2 = rng.standard_normal((2, 1, 2, 4, 5))
    xs1, xs2 = rng.standard_normal((2, 1, 6, 4, 5))
    w1, w2 = rng.standard_normal((2, 3, 3, 3, 5))
    a, b = 0.75, -1.5
    f = lambda xf, xs, w: oracle.patch_conv3x3_halo(geom, 5, 3, xf, xs, w)
    np.testing.assert_allclose(f(a * xf1 + b * xf2, a * xs1 + b * xs2, w1),
                               a * f(xf1, xs1, w1) + b * f(xf2, xs2, w1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f(xf1, xs1, a * w1 + b * w2),
                               a * f(xf1, xs1, w1) + b * f(xf1, xs1, w2), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("patch", [0, 2])
def test_edge_patches_have_zero_halo(patch):
    """Patch 0 has nothing above, patch n-1 nothing below: the conv equals the
    same conv with the whole stale map outside the one real halo row zeroed."""
    geom = (1, 6, 4, 3, patch)
    rng = np.random.default_rng(11 + patch)
    xf, xs = rng.standard_normal((1, 2, 4, 5)), rng.standard_normal((1, 6, 4, 5))
    w = rng.standard_normal((3, 3, 3, 5))
    ref = libref.conv_ref(geom, xf, xs, w)
    got = oracle.patch_conv3x3_halo(geom, 5, 3, xf, xs, w)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the far halo row sits outside the image: perturbing every stale row that
    # is not the single neighbour row must change nothing
    keep = 2 if patch == 0 else 3
    xs2 = np.full_like(xs, np.nan)
    xs2[:, keep] = xs[:, keep]
    np.testing.assert_array_equal(oracle.patch_conv3x3_halo(geom, 5, 3, xf, xs2, w), got)


def test_nan_poison_in_unread_regions():
    wl, d = _inputs("tiny", 1)
    geom = wl.geom
    scale = 0.125
    base = oracle.patch_self_attn(geom, 2, 64, scale, d["q"], d["k_fresh"], d["v_fresh"],
                                  d["k_stale"], d["v_stale"], rows=(0, 64))
    ks = d["k_stale"].double().numpy().copy()
    vs = d["v_stale"].double().numpy().copy()
    ks[:, 512:1024] = np.nan  # patch 1's own tokens in the stale map
    vs[:, 512:1024] = np.nan
    pois = oracle.patch_self_attn(geom, 2, 64, scale, d["q"], d["k_fresh"], d["v_fresh"], ks, vs, rows=(0, 64))
    np.testing.assert_array_equal(pois, base)

    y0 = oracle.patch_conv3x3_halo(geom, 128, 128, d["x_fresh"], d["x_stale"], d["weight"], d["bias"])
    xs = np.full(d["x_stale"].shape, np.nan)
    xs[:, 15] = d["x_stale"][:, 15].double().numpy()  # the only stale row patch 1 may read
    y1 = oracle.patch_conv3x3_halo(geom, 128, 128, d["x_fresh"], xs, d["weight"], d["bias"])
    np.testing.assert_array_equal(y1, y0)

    table = libref.patch_moments(d["x_stale"], geom, 32)
    g0, _ = oracle.async_groupnorm(geom, 128, 32, 1e-5, d["x_fresh"], table, d["gamma"], d["beta"])
    table[:, 1] = np.nan
    g1, _ = oracle.async_groupnorm(geom, 128, 32, 1e-5, d["x_fresh"], table, d["gamma"], d["beta"])
    np.testing.assert_array_equal(g1, g0)


def test_refresh_replaces_only_the_patch_rows():
    rng = np.random.default_rng(2)
    B, H, n, i, E = 2, 12, 4, 2, 7
    stale = rng.standard_normal((B, H, E))
    fresh = rng.standard_normal((B, 3, E))
    out = oracle.refresh_stale((B, H, 1, n, i), E, fresh, stale)
    ref = stale.copy()
    ref[:, 6:9] = fresh
    np.testing.assert_array_equal(out, ref)


def test_moments_match_numpy():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 5, 12)) + 0.5
    m = oracle.group_moments(x, 3)
    g = x.reshape(2, 15, 3, 4)
    np.testing.assert_allclose(m[..., 0], g.mean(axis=(1, 3)), rtol=1e-13)
    np.testing.assert_allclose(m[..., 1], (g ** 2).mean(axis=(1, 3)), rtol=1e-13)


def test_oracle_rejects_bad_geometry():
    x = np.zeros((1, 1, 1, 1, 1))
    with pytest.raises(ValueError):
        oracle.patch_self_attn((1, 5, 1, 2, 0), 1, 1, 1.0, x, x, x, x, x)
    with pytest.raises(ValueError):
        oracle.async_groupnorm((1, 2, 1, 2, 2), 2, 1, 0.0, np.zeros((1, 1, 1, 2)), np.zeros((1, 2, 1, 2)))


def test_thread_count_changes_no_result():
    """Every output element is computed by one thread in a fixed order, so the
    oracle's results are the same bits on one host thread as on all of them
    (the benchmark times it both ways)."""
    wl = si.WORKLOADS["tiny"].with_patch(1)
    d = {k: v.double().numpy() for k, v in si.make_inputs(wl, device="cpu", nonzero_bias=True).items()}
    B, n, G, h = wl.batch, wl.n_patches, wl.groups, wl.h
    table = np.stack([oracle.group_moments(d["x_stale"][:, j * h:(j + 1) * h], G) for j in range(n)], axis=1)

    def run():
        a = oracle.patch_self_attn(wl.geom, wl.heads, 64, wl.head_dim ** -0.5, d["q"], d["k_fresh"],
                                   d["v_fresh"], d["k_stale"], d["v_stale"])
        c = oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, d["x_fresh"], d["x_stale"],
                                      d["weight"], d["bias"])
        g, fm = oracle.async_groupnorm(wl.geom, wl.channels, G, wl.eps, d["x_fresh"], table, d["gamma"],
                                       d["beta"])
        return a, c, g, fm

    before = oracle.num_threads()
    try:
        many = run()
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        one = run()
    finally:
        oracle.set_num_threads(before)
    assert oracle.num_threads() == before
    for x, y in zip(many, one):
        assert np.array_equal(x, y)
