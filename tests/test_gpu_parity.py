"""GPU parity: every op through the C ABI against the CPU oracle on the same
seeded inputs (tolerances in tests/parity_util.py).

Small workloads are compared element by element over the whole output; the
2048^2 and 3840^2 workloads run the kernels at full size, in the launch
configuration the benchmark times, and compare sampled output rows that the
oracle computes one by one (first rows, a tile boundary, the ragged tail).
"""
import math

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
    dp.load()  # raises if the HIP library is missing


W = si.WORKLOADS
RAGGED_BF16 = si.Workload("ragged_bf16", 1, 128, 20, 13, 4, 2, seed=2024)     # Lq=65, L=260
RAGGED_F32 = si.Workload("ragged_f32", 2, 64, 12, 7, 3, 1, dtype="f32", sigma=0.05, seed=2025)
# one partial key tile (L = 32) and 16 queries: a single task, seven idle waves
TINY_L_BF16 = si.Workload("tiny_l_bf16", 1, 128, 4, 8, 2, 2, seed=2026)          # Lq=16, L=32
# one full 512-query tile plus a partial one (88 queries), 3 heads, L = 600
TAIL_BF16 = si.Workload("tail_bf16", 1, 192, 30, 20, 1, 3, seed=2027)            # Lq=L=600
FULL_CASES = [(W["tiny"], 0), (W["tiny"], 1), (W["sdxl1024_l2"], 0), (W["sdxl1024_l2"], 3),
              (W["sdxl1024_l2"], 7), (W["sdxl1024_l3"], 1), (W["sdxl1024_l3"], 3),
              (RAGGED_BF16, 0), (RAGGED_BF16, 2), (RAGGED_BF16, 3), (RAGGED_F32, 1),
              (TINY_L_BF16, 1), (TAIL_BF16, 0)]
SAMPLED_CASES = [(W["sdxl2048_l2"], 0), (W["sdxl2048_l2"], 4), (W["sdxl2048_l2"], 7),
                 (W["sdxl3840_l2"], 0), (W["sdxl3840_l2"], 4), (W["sdxl3840_l2"], 7),
                 (W["sdxl3840_l3"], 0), (W["sdxl3840_l3"], 4), (W["sdxl3840_l3"], 7)]


def _ids(cases):
    return [f"{wl.name}-p{i}" for wl, i in cases]


def _run_attention(wl, g):
    return dp.distri_patch_self_attn(wl.geom, wl.heads, g["q"], g["k_fresh"], g["v_fresh"],
                                     g["k_stale"], g["v_stale"], scale=wl.head_dim ** -0.5)


def _oracle_attention(wl, d, rows=None):
    return oracle.patch_self_attn(wl.geom, wl.heads, wl.head_dim, wl.head_dim ** -0.5, d["q"],
                                  d["k_fresh"], d["v_fresh"], d["k_stale"], d["v_stale"], rows=rows)


@pytest.mark.parametrize("wl,patch", FULL_CASES, ids=_ids(FULL_CASES))
def test_all_ops_full_output(wl, patch):
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    tag = f"{wl.name} patch {patch}"

    out = _run_attention(wl, g)
    assert_close(to_np(out), _oracle_attention(wl, d), wl.dtype, f"attention {tag}")

    y = dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"], g["bias"])
    ref = oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, d["x_fresh"], d["x_stale"],
                                    d["weight"], d["bias"])
    assert_close(to_np(y), ref, wl.dtype, f"conv {tag}")

    yg, fm = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"],
                                       g["beta"], eps=wl.eps)
    ref_y, ref_fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                           d["table"].double().numpy(), d["gamma"], d["beta"])
    assert_close(to_np(yg), ref_y, wl.dtype, f"groupnorm {tag}")
    fmn = to_np(fm)
    assert np.all(np.abs(fmn[..., 0] - ref_fm[..., 0]) <= 1e-5 * np.sqrt(ref_fm[..., 1]) + 1e-7)
    assert np.all(np.abs(fmn[..., 1] - ref_fm[..., 1]) <= 1e-5 * ref_fm[..., 1] + 1e-7)


@pytest.mark.parametrize("wl,patch", SAMPLED_CASES, ids=_ids(SAMPLED_CASES))
def test_full_size_sampled(wl, patch):
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    tag = f"{wl.name} patch {patch}"
    out = to_np(_run_attention(wl, g))
    for r0, r1 in sample_rows(wl.lq, 256, 4):
        ref = _oracle_attention(wl, d, rows=(r0, r1))
        assert_close(out[:, r0:r1], ref, wl.dtype, f"attention {tag} rows {r0}:{r1}")

    y = to_np(dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"], g["bias"]))
    for r0, r1 in [(0, 1), (wl.h // 2, wl.h // 2 + 1), (wl.h - 1, wl.h)]:
        ref = oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, d["x_fresh"], d["x_stale"],
                                        d["weight"], d["bias"], rows=(r0, r1))
        assert_close(y[:, r0:r1], ref, wl.dtype, f"conv {tag} rows {r0}:{r1}")

    yg, fm = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"],
                                       g["beta"], eps=wl.eps)
    ref_y, ref_fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                           d["table"].double().numpy(), d["gamma"], d["beta"])
    assert_close(to_np(yg), ref_y, wl.dtype, f"groupnorm {tag}")
    np.testing.assert_allclose(to_np(fm), ref_fm, rtol=1e-5, atol=1e-7)


REFRESH_CASES = [(W["tiny"], 1), (W["sdxl1024_l2"], 5), (W["sdxl3840_l2"], 4), (RAGGED_BF16, 3)]


@pytest.mark.parametrize("wl,patch", REFRESH_CASES, ids=_ids(REFRESH_CASES))
def test_refresh_bitwise(wl, patch):
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    B, H, Wd, h = wl.batch, wl.height, wl.width, wl.h
    tok_row = Wd * wl.heads * wl.head_dim
    for fresh, stale, row in (("k_fresh", "k_stale", tok_row), ("v_fresh", "v_stale", tok_row),
                              ("x_fresh", "x_stale", Wd * wl.channels)):
        s = g[stale].clone()
        dp.distri_refresh_stale(wl.geom, row, g[fresh], s)
        ref = d[stale].clone()
        ref.view(B, H, row)[:, patch * h:(patch + 1) * h] = d[fresh].view(B, h, row)
        assert torch.equal(s.cpu().view(torch.int16 if s.dtype == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if s.dtype == torch.bfloat16 else torch.int32))
    # the GroupNorm moment table: geometry (B, n, 1, n, i), 2G floats per row
    tab = g["table"].clone()
    fresh_m = torch.randn(B, wl.groups, 2).cuda()
    dp.distri_refresh_stale((B, wl.n_patches, 1, wl.n_patches, patch), 2 * wl.groups, fresh_m, tab)
    ref = d["table"].clone()
    ref[:, patch] = fresh_m.cpu()
    assert torch.equal(tab.cpu(), ref)


MAPS_CASES = [(W["tiny"], 1), (W["sdxl3840_l2"], 0), (W["sdxl3840_l3"], 7), (RAGGED_BF16, 3),
              (W["sdxl3840_l2"], 4)]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("wl,patch", MAPS_CASES, ids=_ids(MAPS_CASES))
def test_refresh_maps_bitwise(wl, patch):
    """All of a layer's maps in one call (K, V, the conv input, the moment
    table, and a map of 6-byte rows that takes a launch of its own): patch
    rows replaced bit for bit, every other row untouched."""
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    B, H, Wd, h, n = wl.batch, wl.height, wl.width, wl.h, wl.n_patches
    tok_row = Wd * wl.heads * wl.head_dim
    odd_f = torch.arange(B * h * 3, dtype=torch.float32).to(torch.bfloat16).cuda()
    odd_s = torch.full((B * H * 3,), -1.0, dtype=torch.bfloat16).cuda()
    fresh_m = torch.randn(B, wl.groups, 2).cuda()
    maps = [(h, tok_row, g["k_fresh"], g["k_stale"].clone()), (h, tok_row, g["v_fresh"], g["v_stale"].clone()),
            (h, Wd * wl.channels, g["x_fresh"], g["x_stale"].clone()), (1, 2 * wl.groups, fresh_m, g["table"].clone()),
            (h, 3, odd_f, odd_s)]
    before = [m[3].cpu() for m in maps]
    dp.distri_refresh_stale_maps(wl.geom, maps)
    torch.cuda.synchronize()
    for (rows, row, fresh, stale), old in zip(maps, before):
        ref = old.clone().view(B, n * rows, row)
        ref[:, patch * rows:(patch + 1) * rows] = fresh.cpu().view(B, rows, row)
        assert torch.equal(_bits(stale.cpu().view(B, n * rows, row)), _bits(ref)), (rows, row)


def test_refresh_maps_matches_single_map_calls():
    """The one-launch form and one distri_refresh_stale per map leave the
    same bytes (three images; per-image ranges whose sizes are off any
    64 KiB boundary, so chunks end inside a range)."""
    geom = (3, 40, 24, 5, 2)
    B, H, Wd, n, i = geom
    h = H // n
    gen = torch.Generator(device="cuda").manual_seed(3)
    maps_a, maps_b = [], []
    for row in (Wd * 8, Wd * 1000, 16):
        fresh = torch.randn(B, h, row, generator=gen, device="cuda").to(torch.bfloat16)
        stale = torch.randn(B, H, row, generator=gen, device="cuda").to(torch.bfloat16)
        maps_a.append((h, row, fresh, stale.clone()))
        dp.distri_refresh_stale(geom, row, fresh, stale)
        maps_b.append(stale)
    dp.distri_refresh_stale_maps(geom, maps_a)
    torch.cuda.synchronize()
    for (_, _, _, got), want in zip(maps_a, maps_b):
        assert torch.equal(_bits(got), _bits(want))


@pytest.mark.parametrize("cout", [200, 90, 8, 160], ids=["cout200", "cout90", "cout8", "cout160"])
def test_conv_output_channel_counts(cout):
    """Cout other than Cin: a partial 160-channel tile (200), a count that is
    not a multiple of 8 (90: element stores instead of the staged 16-byte
    ones), a tile of 8 channels, and exactly one tile."""
    geom = (2, 12, 11, 3, 1)
    B, H, Wd, n, i = geom
    h, cin = H // n, 64
    gen = torch.Generator().manual_seed(4100 + cout)
    xf = torch.randn(B, h, Wd, cin, generator=gen).to(torch.bfloat16)
    xs = torch.randn(B, H, Wd, cin, generator=gen).to(torch.bfloat16)
    w = (torch.randn(cout, 3, 3, cin, generator=gen) / 24.0).to(torch.bfloat16)
    bias = 0.1 * torch.randn(cout, generator=gen)
    y = dp.distri_patch_conv3x3_halo(geom, xf.cuda(), xs.cuda(), w.cuda(), bias.cuda())
    ref = oracle.patch_conv3x3_halo(geom, cin, cout, xf, xs, w, bias)
    assert_close(to_np(y), ref, "bf16", f"conv cout {cout}")


def test_refresh_odd_rows_and_alignment():
    """Rows whose byte size is not a multiple of 16 (scalar path)."""
    geom = (3, 6, 1, 3, 1)
    fresh = torch.arange(3 * 2 * 5, dtype=torch.bfloat16).cuda()
    stale = torch.full((3 * 6 * 5,), -1.0, dtype=torch.bfloat16).cuda()
    dp.distri_refresh_stale(geom, 5, fresh, stale)
    ref = torch.full((3, 6, 5), -1.0, dtype=torch.bfloat16)
    ref[:, 2:4] = fresh.cpu().view(3, 2, 5)
    assert torch.equal(stale.cpu().view(3, 6, 5), ref)


def test_stale_equals_fresh_matches_oracle():
    wl = W["sdxl1024_l3"].with_patch(2)
    d = cpu_inputs(wl, stale_equals_fresh=True)
    g = gpu_copy(d)
    assert_close(to_np(_run_attention(wl, g)), _oracle_attention(wl, d), "bf16", "attention stale=fresh")
    y = dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"], g["bias"])
    ref = oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, d["x_fresh"], d["x_stale"],
                                    d["weight"], d["bias"])
    assert_close(to_np(y), ref, "bf16", "conv stale=fresh")


def test_nan_poison_of_unread_regions_changes_nothing():
    wl = RAGGED_BF16.with_patch(2)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    base_attn = _run_attention(wl, g)
    base_conv = dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"], g["bias"])
    base_gn, _ = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"],
                                           g["beta"])
    lo, hi = 2 * wl.lq, 3 * wl.lq
    p = dict(g)
    p["k_stale"] = g["k_stale"].clone()
    p["v_stale"] = g["v_stale"].clone()
    p["k_stale"][:, lo:hi] = float("nan")
    p["v_stale"][:, lo:hi] = float("nan")
    xs = torch.full_like(g["x_stale"], float("nan"))
    h = wl.h
    xs[:, 2 * h - 1] = g["x_stale"][:, 2 * h - 1]
    xs[:, 3 * h] = g["x_stale"][:, 3 * h]
    tab = g["table"].clone()
    tab[:, 2] = float("nan")
    assert torch.equal(_run_attention(wl, p), base_attn)
    assert torch.equal(dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], xs, g["weight"], g["bias"]),
                       base_conv)
    assert torch.equal(dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], tab, g["gamma"],
                                                 g["beta"])[0], base_gn)


def test_guard_regions_untouched_and_deterministic():
    wl = RAGGED_BF16.with_patch(1)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    n_out = g["q"].numel()
    guard = 4096
    buf = torch.full((n_out + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[guard:guard + n_out].view(g["q"].shape)
    dp.distri_patch_self_attn(wl.geom, wl.heads, g["q"], g["k_fresh"], g["v_fresh"], g["k_stale"],
                              g["v_stale"], out=out)
    again = _run_attention(wl, g)
    torch.cuda.synchronize()
    assert torch.all(buf[:guard] == 7.0) and torch.all(buf[guard + n_out:] == 7.0)
    assert torch.equal(out, again)
    n_y = g["x_fresh"].numel()
    buf = torch.full((n_y + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    y = buf[guard:guard + n_y].view(g["x_fresh"].shape)
    dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"], g["bias"], y=y)
    assert torch.all(buf[:guard] == 7.0) and torch.all(buf[guard + n_y:] == 7.0)
    assert torch.equal(y, dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], g["x_stale"], g["weight"],
                                                       g["bias"]))
    buf = torch.full((n_y + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    yg = buf[guard:guard + n_y].view(g["x_fresh"].shape)
    dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"], g["beta"], y=yg)
    assert torch.all(buf[:guard] == 7.0) and torch.all(buf[guard + n_y:] == 7.0)


def test_single_patch_needs_no_stale_map():
    wl = si.Workload("one_patch", 2, 64, 8, 8, 1, 1, seed=99)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    y = dp.distri_patch_conv3x3_halo(wl.geom, g["x_fresh"], None, g["weight"], g["bias"])
    ref = oracle.patch_conv3x3_halo(wl.geom, 64, 64, d["x_fresh"], d["x_stale"], d["weight"], d["bias"])
    assert_close(to_np(y), ref, "bf16", "conv n=1")
    out = _run_attention(wl, g)
    assert_close(to_np(out), _oracle_attention(wl, d), "bf16", "attention n=1")


def test_empty_batch_is_a_no_op():
    geom = (0, 8, 8, 2, 0)
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    dp.distri_patch_self_attn(geom, 1, e, e, e, e, e, out=e)
    dp.distri_refresh_stale(geom, 64, e, e)
    torch.cuda.synchronize()


def test_extreme_scores_stay_finite():
    """Large-magnitude logits: the online softmax must rescale correctly."""
    wl = si.Workload("hot", 1, 64, 16, 16, 2, 1, seed=7)
    d = cpu_inputs(wl)
    d = dict(d)
    d["q"] = (d["q"].float() * 6).to(torch.bfloat16)
    g = gpu_copy(d)
    out = _run_attention(wl, g)
    assert_close(to_np(out), _oracle_attention(wl, d), "bf16", "attention large logits")


# GroupNorm launch shapes away from the SDXL ones: groups that split a
# 16-byte channel vector (C/G = 4), one group, block widths that are not a
# power of two (C = 40 -> 5 vectors per pixel), fp32, and more chunks than
# one block row covers.  The last two take the three-launch form: more than
# 256 images (the single-launch form holds at most 192 blocks, one image or
# more per block), and a slice of more than 32 pixels per thread at 256
# blocks.
GN_SHAPES = [si.Workload("gn_c40_g5", 2, 40, 12, 10, 3, 1, groups=5, seed=3001, patch=1),
             si.Workload("gn_c1024_g256", 1, 1024, 8, 6, 2, 1, groups=256, seed=3002, patch=1),
             si.Workload("gn_c64_g1", 3, 64, 16, 9, 4, 1, groups=1, seed=3003, patch=3),
             si.Workload("gn_f32_c12_g3", 2, 12, 10, 11, 5, 1, groups=3, dtype="f32", sigma=0.05,
                         seed=3004, patch=2),
             si.Workload("gn_c2048_g32", 3, 2048, 32, 24, 4, 1, groups=32, seed=3005, patch=0),
             si.Workload("gn_b257_three_launch", 257, 32, 8, 8, 2, 1, groups=8, seed=3006, patch=1),
             si.Workload("gn_big_slice_three_launch", 1, 1024, 184, 184, 1, 1, groups=32, seed=3007)]


@pytest.mark.parametrize("wl", GN_SHAPES, ids=[w.name for w in GN_SHAPES])
def test_groupnorm_shapes(wl):
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    yg, fm = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"],
                                       g["beta"], eps=wl.eps)
    ref_y, ref_fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                           d["table"].double().numpy(), d["gamma"], d["beta"])
    assert_close(to_np(yg), ref_y, wl.dtype, f"groupnorm {wl.name}")
    fmn = to_np(fm)
    assert np.all(np.abs(fmn[..., 0] - ref_fm[..., 0]) <= 1e-5 * np.sqrt(ref_fm[..., 1]) + 1e-7)
    assert np.all(np.abs(fmn[..., 1] - ref_fm[..., 1]) <= 1e-5 * ref_fm[..., 1] + 1e-7)


def test_groupnorm_reused_workspace_is_exact():
    """The GroupNorm workspace carries per-call flags between its two
    launches; reusing one workspace (also after filling it with arbitrary
    bytes) across calls on different inputs must give the same bits as a
    fresh zeroed workspace each time."""
    wl = W["sdxl1024_l2"].with_patch(3)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    nb = dp.distri_async_groupnorm_workspace_size(wl.geom, wl.channels, wl.groups, dp.DISTRI_BF16)
    shared = torch.randint(0, 255, (nb,), dtype=torch.uint8, device="cuda")
    for k in range(3):
        x = (g["x_fresh"].float() * (1.0 + 0.5 * k) + 0.25 * k).to(torch.bfloat16)
        ref_y, ref_fm = dp.distri_async_groupnorm(
            wl.geom, wl.groups, x, g["table"], g["gamma"], g["beta"],
            workspace=torch.zeros(nb, dtype=torch.uint8, device="cuda"))
        y, fm = dp.distri_async_groupnorm(wl.geom, wl.groups, x, g["table"], g["gamma"], g["beta"],
                                          workspace=shared)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16)), f"call {k}"
        assert torch.equal(fm, ref_fm), f"call {k}"


def test_groupnorm_workspace_shared_across_shapes():
    """One workspace serves, in turn, GroupNorms of different shapes (so of
    different block counts, with flags of one shape's calls left where the
    other shape's blocks look) and the moments-only, normalise and SiLU
    forms; every call must give the bits of a call on a zeroed workspace."""
    wls = [W["sdxl1024_l2"].with_patch(3), W["sdxl1024_l3"].with_patch(0), W["tiny"].with_patch(1)]
    ins = [(wl, gpu_copy(cpu_inputs(wl))) for wl in wls]
    nb = max(dp.distri_async_groupnorm_workspace_size(wl.geom, wl.channels, wl.groups,
                                                      dp.DISTRI_BF16 if wl.dtype == "bf16" else dp.DISTRI_F32)
             for wl in wls)
    shared = torch.randint(0, 255, (nb,), dtype=torch.uint8, device="cuda")
    for k in range(7):
        wl, g = ins[k % len(ins)]
        fn = dp.distri_async_groupnorm_silu if k % 2 else dp.distri_async_groupnorm
        ref_y, ref_fm = fn(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"], g["beta"],
                           eps=wl.eps, workspace=torch.zeros(nb, dtype=torch.uint8, device="cuda"))
        y, fm = fn(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"], g["beta"], eps=wl.eps,
                   workspace=shared)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16 if wl.dtype == "bf16" else torch.int32),
                           ref_y.view(torch.int16 if wl.dtype == "bf16" else torch.int32)), f"call {k}"
        assert torch.equal(fm, ref_fm), f"call {k}"


@pytest.mark.parametrize("v_scale", [2.0 ** 12, 2.0 ** -10], ids=["v_x4096", "v_x2^-10"])
def test_attention_value_range(v_scale):
    """The weighted sum of V runs in f16: V far above and below unit scale
    (|v| up to about 2e4, and down into f16's subnormal range) still meets
    the bound."""
    wl = W["sdxl1024_l3"].with_patch(2)
    d = dict(cpu_inputs(wl))
    for k in ("v_fresh", "v_stale"):
        d[k] = (d[k].float() * v_scale).to(torch.bfloat16)
    g = gpu_copy(d)
    assert_close(to_np(_run_attention(wl, g)), _oracle_attention(wl, d), "bf16",
                 f"attention V x {v_scale:g}")
