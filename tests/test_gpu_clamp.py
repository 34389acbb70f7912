"""GPU parity of the corrected asynchronous GroupNorm when the variance clamp
acts.

The stale moments of the other patches are made inconsistent with the fresh
slice: on even groups every other patch reports E[x] = 2 and E[x^2] = 0.5,
so after the equal-weight mix E[x^2] - E[x]^2 is negative and the variance is
clamped to 0 (rstd = 1 / sqrt(eps)); odd groups keep ordinary moments.  The
kernels are compared with the oracle, whose clamp is pinned on the CPU to the
closed form (x - mu) / sqrt(eps) gamma + beta.  Each case first checks, from
the oracle's own fresh moments, that the clamp really acts on the even groups
and not on the odd ones.
"""
import dataclasses

import numpy as np
import pytest
import torch

import displaced_patch_parallelism_distri_amd as dp
import oracle
import synthetic_inputs as si
from tests.parity_util import assert_close, cpu_inputs, gpu_copy, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()


def clamping_table(B, n, G, seed):
    """[B, n, G, 2] fp32: even groups (2, 0.5), odd groups (0.1 N, m1^2 + U(0.5, 1.5))."""
    gen = torch.Generator().manual_seed(seed)
    m1 = 0.1 * torch.randn(B, n, G, generator=gen)
    m2 = m1 * m1 + 0.5 + torch.rand(B, n, G, generator=gen)
    m1[:, :, 0::2] = 2.0
    m2[:, :, 0::2] = 0.5
    return torch.stack([m1, m2], dim=-1).float().contiguous()


def mixed_variance(fresh, table, i):
    """E[x^2] - E[x]^2 of the equal-weight mix of slot i's fresh moments with
    the other slots of the table (fp64), [B, G]."""
    t = np.asarray(table, dtype=np.float64).copy()
    t[:, i] = fresh
    mu = t[..., 0].mean(axis=1)
    e2 = t[..., 1].mean(axis=1)
    return e2 - mu * mu


def assert_clamps_even_groups_only(var, what):
    assert np.all(var[:, 0::2] < 0), f"{what}: the clamp does not act on every even group"
    assert np.all(var[:, 1::2] > 0), f"{what}: an odd group is clamped too"


CASES = [(si.WORKLOADS["sdxl1024_l2"], 3), (si.WORKLOADS["sdxl1024_l3"], 0),
         (si.WORKLOADS["tiny"], 1), (si.WORKLOADS["sdxl3840_l3"], 7)]


@pytest.mark.parametrize("wl,patch", CASES, ids=[f"{w.name}-p{i}" for w, i in CASES])
def test_groupnorm_clamp(wl, patch):
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    table = clamping_table(wl.batch, wl.n_patches, wl.groups, wl.seed + 77)
    ref_y, ref_fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                           table.double().numpy(), d["gamma"], d["beta"])
    assert_clamps_even_groups_only(mixed_variance(ref_fm, table, patch), wl.name)
    tg = table.cuda()
    y, fm = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], tg, g["gamma"], g["beta"],
                                      eps=wl.eps)
    assert_close(to_np(y), ref_y, wl.dtype, f"clamped groupnorm {wl.name} patch {patch}")
    np.testing.assert_allclose(to_np(fm), ref_fm, rtol=1e-5, atol=1e-7)
    ys, _ = dp.distri_async_groupnorm_silu(wl.geom, wl.groups, g["x_fresh"], tg, g["gamma"],
                                           g["beta"], eps=wl.eps)
    assert_close(to_np(ys), oracle.silu(ref_y), wl.dtype,
                 f"clamped groupnorm+silu {wl.name} patch {patch}")


# The block with both GroupNorm tables clamping.  eps = 1 keeps the clamped
# normalisation at rstd = 1, so the activations that reach attention stay of
# order one (with eps = 1e-5 the clamped groups are scaled by 316 and the
# softmax of the block becomes ill-conditioned, which would test the inputs,
# not the kernels).
BLOCK_CASES = [(dataclasses.replace(si.Workload("block_clamp", 2, 256, 32, 32, 4, 4, seed=5301), eps=1.0), 1),
               (dataclasses.replace(si.Workload("block_clamp_f32", 1, 128, 12, 7, 3, 2, groups=16,
                                                dtype="f32", sigma=0.05, seed=5302), eps=1.0), 2)]


@pytest.mark.parametrize("wl,patch", BLOCK_CASES, ids=[f"{w.name}-p{i}" for w, i in BLOCK_CASES])
def test_block_clamp(wl, patch):
    wl = wl.with_patch(patch)
    d = si.make_block_inputs(wl)
    st = dict(d["state"])
    st["gn1"] = clamping_table(wl.batch, wl.n_patches, wl.groups, wl.seed + 1)
    st["gn2"] = clamping_table(wl.batch, wl.n_patches, wl.groups, wl.seed + 2)
    wts = dict(si.block_scalars(wl))
    wts.update({k: v.double().numpy() for k, v in d["weights"].items()})
    h = wl.h
    x_cpu = d["x"][:, patch * h:(patch + 1) * h].contiguous()
    ref_y, ref_st = oracle.patch_block(wl.geom, wts, x_cpu, st, act_dtype=wl.dtype)
    for key in ("gn1", "gn2"):
        assert_clamps_even_groups_only(mixed_variance(ref_st[key][:, patch], st[key], patch),
                                       f"{wl.name} {key}")
    gst = {k: v.cuda().clone() for k, v in st.items()}
    gw = {k: v.cuda() for k, v in d["weights"].items()}
    y = dp.distri_patch_block(wl.geom, gw, x_cpu.cuda(), gst, groups=wl.groups, heads=wl.heads,
                              eps=wl.eps, scale=wl.head_dim ** -0.5)
    assert_close(to_np(y), ref_y, wl.dtype, f"clamped block {wl.name} patch {patch}")
    i, Lq = patch, wl.lq
    assert_close(to_np(gst["conv_in"][:, i * h:(i + 1) * h]), ref_st["conv_in"][:, i * h:(i + 1) * h],
                 wl.dtype, f"clamped block {wl.name} state conv_in")
    assert_close(to_np(gst["k"][:, i * Lq:(i + 1) * Lq]), ref_st["k"][:, i * Lq:(i + 1) * Lq],
                 wl.dtype, f"clamped block {wl.name} state k")
