"""GPU parity of the attention layer's projections (Q/K/V with the fused
refresh of the stale K/V maps, and the output projection) through the C ABI,
against the CPU oracle on the same seeded inputs (tolerance rule in
tests/parity_util.py).  The stale maps must hold, in the patch's rows, exactly
the bits of the fresh K / V the call returned, and elsewhere exactly what they
held before.
"""
import numpy as np
import pytest
import torch

import displaced_patch_parallelism_distri_amd as dp
import oracle
import synthetic_inputs as si
from tests.parity_util import assert_close, sample_rows, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()


W = si.WORKLOADS
C64_BF16 = si.Workload("proj_c64_bf16", 3, 64, 10, 9, 2, 1, seed=4101)       # N = 192: ragged N tile
RAGGED_BF16 = si.Workload("proj_ragged_bf16", 1, 128, 20, 13, 4, 2, seed=4102)  # M = 65
RAGGED_F32 = si.Workload("proj_ragged_f32", 2, 96, 12, 7, 3, 1, dtype="f32", seed=4103)
FULL_CASES = [(W["tiny"], 1), (W["sdxl1024_l2"], 3), (W["sdxl1024_l3"], 1), (C64_BF16, 1),
              (RAGGED_BF16, 3), (RAGGED_F32, 2)]
SAMPLED_CASES = [(W["sdxl3840_l2"], 4), (W["sdxl3840_l3"], 7)]


def _ids(cases):
    return [f"{wl.name}-p{i}" for wl, i in cases]


def _bits(t):
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _check_stale(wl, before, after, fresh, what):
    """Patch rows of ``after`` carry the bits of ``fresh``; the rest is
    ``before`` unchanged."""
    i, Lq = wl.patch, wl.lq
    a, b = _bits(after), _bits(before)
    assert torch.equal(a[:, i * Lq:(i + 1) * Lq], _bits(fresh)), f"{what}: patch rows != fresh"
    assert torch.equal(a[:, :i * Lq], b[:, :i * Lq]), f"{what}: rows before the patch changed"
    assert torch.equal(a[:, (i + 1) * Lq:], b[:, (i + 1) * Lq:]), f"{what}: rows after the patch changed"


@pytest.mark.parametrize("wl,patch", FULL_CASES, ids=_ids(FULL_CASES))
def test_qkv_and_out_proj_full_output(wl, patch):
    wl = wl.with_patch(patch)
    d = si.make_proj_inputs(wl)
    g = {k: v.cuda() for k, v in d.items()}
    tag = f"{wl.name} patch {patch}"
    ks, vs = g["k_stale"].clone(), g["v_stale"].clone()
    q, k, v = dp.distri_patch_qkv_proj(wl.geom, g["x"], g["w_qkv"], g["b_qkv"], k_stale=ks, v_stale=vs)
    rq, rk, rv, _, _ = oracle.patch_qkv_proj(wl.geom, wl.channels, d["x"], d["w_qkv"], d["b_qkv"])
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(to_np(got), ref, wl.dtype, f"qkv_proj {name} {tag}")
    _check_stale(wl, d["k_stale"], ks, k, f"k_stale {tag}")
    _check_stale(wl, d["v_stale"], vs, v, f"v_stale {tag}")

    y = dp.distri_patch_out_proj(wl.geom, g["o"], g["w_o"], g["b_o"])
    assert_close(to_np(y), oracle.linear(d["o"], d["w_o"], d["b_o"]), wl.dtype, f"out_proj {tag}")


def test_qkv_without_stale_maps_or_bias():
    wl = W["sdxl1024_l2"].with_patch(6)
    d = si.make_proj_inputs(wl)
    g = {k: v.cuda() for k, v in d.items()}
    q, k, v = dp.distri_patch_qkv_proj(wl.geom, g["x"], g["w_qkv"])
    rq, rk, rv, _, _ = oracle.patch_qkv_proj(wl.geom, wl.channels, d["x"], d["w_qkv"])
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(to_np(got), ref, wl.dtype, f"qkv_proj {name} no bias")
    # with the stale maps the returned q/k/v are the same bits
    ks = g["k_stale"].clone()
    q2, k2, v2 = dp.distri_patch_qkv_proj(wl.geom, g["x"], g["w_qkv"], k_stale=ks)
    for a, b in ((q, q2), (k, k2), (v, v2)):
        assert torch.equal(_bits(a), _bits(b))
    _check_stale(wl, d["k_stale"], ks, k2, "k_stale only")
    y = dp.distri_patch_out_proj(wl.geom, g["o"], g["w_o"])
    assert_close(to_np(y), oracle.linear(d["o"], d["w_o"]), wl.dtype, "out_proj no bias")


@pytest.mark.parametrize("wl,patch", SAMPLED_CASES, ids=_ids(SAMPLED_CASES))
def test_proj_full_size_sampled(wl, patch):
    wl = wl.with_patch(patch)
    d = si.make_proj_inputs(wl)
    g = {k: v.cuda() for k, v in d.items()}
    tag = f"{wl.name} patch {patch}"
    ks, vs = g["k_stale"].clone(), g["v_stale"].clone()
    q, k, v = dp.distri_patch_qkv_proj(wl.geom, g["x"], g["w_qkv"], g["b_qkv"], k_stale=ks, v_stale=vs)
    y = dp.distri_patch_out_proj(wl.geom, g["o"], g["w_o"], g["b_o"])
    qkv = np.concatenate([to_np(q), to_np(k), to_np(v)], axis=-1)
    yn = to_np(y)
    for r0, r1 in sample_rows(wl.lq, 128, 4):
        ref = oracle.linear(d["x"][:, r0:r1], d["w_qkv"], d["b_qkv"])
        assert_close(qkv[:, r0:r1], ref, wl.dtype, f"qkv_proj {tag} rows {r0}:{r1}")
        ref = oracle.linear(d["o"][:, r0:r1], d["w_o"], d["b_o"])
        assert_close(yn[:, r0:r1], ref, wl.dtype, f"out_proj {tag} rows {r0}:{r1}")
    _check_stale(wl, d["k_stale"], ks, k, f"k_stale {tag}")
    _check_stale(wl, d["v_stale"], vs, v, f"v_stale {tag}")


def test_attention_layer_chain():
    """Q/K/V projection (refreshing the stale maps) -> attention over the
    fresh + stale K/V -> output projection, against the oracle's chain fed,
    like the library's, with each op's result rounded to the activation dtype
    (q, k, v, the refreshed stale maps and the attention output are bf16
    tensors); each op's own result is compared."""
    wl = W["sdxl1024_l2"].with_patch(3)
    d = si.make_proj_inputs(wl)
    g = {k: v.cuda() for k, v in d.items()}
    B, Lq, L, nh, hd = wl.batch, wl.lq, wl.tokens, wl.heads, wl.head_dim
    ks, vs = g["k_stale"].clone(), g["v_stale"].clone()
    q, k, v = dp.distri_patch_qkv_proj(wl.geom, g["x"], g["w_qkv"], g["b_qkv"], k_stale=ks, v_stale=vs)
    o = dp.distri_patch_self_attn(wl.geom, nh, q.view(B, Lq, nh, hd), k.view(B, Lq, nh, hd),
                                  v.view(B, Lq, nh, hd), ks.view(B, L, nh, hd), vs.view(B, L, nh, hd),
                                  scale=hd ** -0.5)
    y = dp.distri_patch_out_proj(wl.geom, o.view(B, Lq, nh * hd), g["w_o"], g["b_o"])

    rq, rk, rv, rks, rvs = oracle.patch_qkv_proj(wl.geom, wl.channels, d["x"], d["w_qkv"], d["b_qkv"],
                                                 d["k_stale"], d["v_stale"])
    sh = (B, Lq, nh, hd)
    r = lambda a: oracle.round_to(a, wl.dtype)
    ro = oracle.patch_self_attn(wl.geom, nh, hd, hd ** -0.5, r(rq).reshape(sh), r(rk).reshape(sh),
                                r(rv).reshape(sh), r(rks).reshape(B, L, nh, hd),
                                r(rvs).reshape(B, L, nh, hd))
    ry = oracle.linear(r(ro).reshape(B, Lq, nh * hd), d["w_o"], d["b_o"])
    assert_close(to_np(o).reshape(B, Lq, -1), ro.reshape(B, Lq, -1), wl.dtype, "chain attention")
    assert_close(to_np(y), ry, wl.dtype, "chain out_proj")
