"""GPU parity of cross-attention with patch queries and of the naive-patch
baseline, through the C ABI, against the CPU oracle (tolerance rule in
tests/parity_util.py).
"""
import numpy as np
import pytest
import torch

import displaced_patch_parallelism_distri_amd as dp
import oracle
import synthetic_inputs as si
from tests.parity_util import assert_close, cpu_inputs, gpu_copy, sample_rows, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()


W = si.WORKLOADS
RAGGED = si.Workload("f4_ragged", 1, 128, 20, 13, 4, 2, seed=5301)     # Lq = 65
RAGGED2 = si.Workload("f4_ragged2", 2, 192, 12, 9, 2, 3, seed=5302)    # Lq = 54, 2 images, 3 heads
# 40 (image, head) pairs x 96 query blocks: the short-context kernel runs
# several query blocks per wave (the next block's Q loaded during this one)
MANY = si.Workload("f4_many_blocks", 2, 1280, 64, 48, 1, 20, seed=5303)  # Lq = 3072
# bf16 contexts of at most 128 tokens take the kernel that holds the whole
# context on chip (1..4 blocks of 32 keys, partial last block); longer ones
# and fp32 take the self-attention kernels
CROSS_CASES = [(W["tiny"], 0, 77), (W["sdxl1024_l2"], 3, 77), (W["sdxl1024_l3"], 1, 77),
               (RAGGED, 2, 5), (RAGGED, 1, 1), (RAGGED, 3, 300), (RAGGED, 0, 32), (RAGGED2, 1, 96),
               (RAGGED2, 0, 17), (W["sdxl1024_l2"], 6, 128), (RAGGED, 1, 129), (MANY, 0, 77)]


@pytest.mark.parametrize("wl,patch,ctx", CROSS_CASES,
                         ids=[f"{w.name}-p{i}-ctx{c}" for w, i, c in CROSS_CASES])
def test_cross_attention(wl, patch, ctx):
    wl = wl.with_patch(patch)
    d = si.make_cross_inputs(wl, ctx)
    g = {k: v.cuda() for k, v in d.items()}
    out = dp.distri_patch_cross_attn(wl.geom, wl.heads, g["q"], g["k_ctx"], g["v_ctx"],
                                     scale=wl.head_dim ** -0.5)
    ref = oracle.cross_attn(wl.head_dim ** -0.5, d["q"], d["k_ctx"], d["v_ctx"])
    assert_close(to_np(out), ref, wl.dtype, f"cross-attention {wl.name} ctx {ctx}")
    if ctx == 1:  # one context token: its V, to the output's rounding
        v = d["v_ctx"].double().numpy()
        assert np.array_equal(to_np(out), np.broadcast_to(v, ref.shape))


@pytest.mark.parametrize("name", ["sdxl3840_l2", "sdxl3840_l3"])
def test_cross_attention_full_size_sampled(name):
    wl = W[name].with_patch(4)
    d = si.make_cross_inputs(wl, 77)
    g = {k: v.cuda() for k, v in d.items()}
    out = to_np(dp.distri_patch_cross_attn(wl.geom, wl.heads, g["q"], g["k_ctx"], g["v_ctx"]))
    for r0, r1 in sample_rows(wl.lq, 256, 4):
        ref = oracle.cross_attn(0.125, d["q"][:, r0:r1], d["k_ctx"], d["v_ctx"])
        assert_close(out[:, r0:r1], ref, wl.dtype, f"cross-attention {name} rows {r0}:{r1}")


NAIVE_CASES = [(W["tiny"], 1), (W["sdxl1024_l2"], 3), (RAGGED, 0)]


@pytest.mark.parametrize("wl,patch", NAIVE_CASES, ids=[f"{w.name}-p{i}" for w, i in NAIVE_CASES])
def test_naive_patch_variant(wl, patch):
    """Each op with the naive geometry (the patch alone) against the oracle's
    layers at n = 1 on the patch rows."""
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    ng = dp.naive_geom(wl.geom)
    ngt = (ng.batch, ng.height, ng.width, 1, 0)
    C, G = wl.channels, wl.groups
    tag = f"naive {wl.name} patch {patch}"
    att = dp.distri_patch_self_attn(ng, wl.heads, g["q"], g["k_fresh"], g["v_fresh"], g["k_fresh"],
                                    g["v_fresh"])
    ref = oracle.patch_self_attn(ngt, wl.heads, 64, 0.125, d["q"], d["k_fresh"], d["v_fresh"], None, None)
    assert_close(to_np(att), ref, wl.dtype, tag + " attention")
    y = dp.distri_patch_conv3x3_halo(ng, g["x_fresh"], None, g["weight"], g["bias"])
    ref = oracle.patch_conv3x3_halo(ngt, C, C, d["x_fresh"], None, d["weight"], d["bias"])
    assert_close(to_np(y), ref, wl.dtype, tag + " conv")
    table = torch.zeros(wl.batch, 1, G, 2, device="cuda")
    yg, _ = dp.distri_async_groupnorm(ng, G, g["x_fresh"], table, g["gamma"], g["beta"], eps=wl.eps)
    ref, _ = oracle.async_groupnorm(ngt, C, G, wl.eps, d["x_fresh"], np.zeros((wl.batch, 1, G, 2)),
                                    d["gamma"], d["beta"])
    assert_close(to_np(yg), ref, wl.dtype, tag + " groupnorm")


def test_naive_conv_seams_are_the_halo_rows_only():
    """Same kernel, two geometries: rows away from the patch boundary are the
    same bits; the rows next to a neighbour differ (the naive seams)."""
    wl = W["sdxl1024_l2"].with_patch(3)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    disp = dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"], g["bias"])
    naive = dp.distri_patch_conv3x3_halo(dp.naive_geom(wl.geom), g["x_fresh"], None, g["weight"],
                                         g["bias"])
    a, b = disp.cpu().view(torch.int16), naive.cpu().view(torch.int16)
    h = wl.h
    assert torch.equal(a[:, 1:h - 1], b[:, 1:h - 1])
    for r in (0, h - 1):
        assert not torch.equal(a[:, r], b[:, r])
