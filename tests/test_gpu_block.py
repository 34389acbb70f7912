"""GPU parity of the patch block (GroupNorm+SiLU -> halo conv -> GroupNorm ->
Q/K/V projection with the K/V refresh -> attention -> output projection) and
of the two GroupNorm forms it adds (SiLU epilogue, moments into the table),
through the C ABI, against the CPU oracle on the same seeded inputs
(tolerance rule in tests/parity_util.py; the block is compared at its output
and at every state map it writes).  The oracle's block is given act_dtype =
the workload dtype: each op reads its inputs as tensors of that dtype, as the
library's chain of ops does, and each op's own result is compared.
"""
import numpy as np
import pytest
import torch

import displaced_patch_parallelism_distri_amd as dp
import oracle
import synthetic_inputs as si
from tests.parity_util import TOL, assert_close, cpu_inputs, gpu_copy, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()


W = si.WORKLOADS
MID = si.Workload("block_mid", 2, 256, 32, 32, 4, 4, seed=5201)                  # Lq = 256, M = 512
RAGGED = si.Workload("block_ragged", 1, 128, 20, 13, 4, 2, seed=5202)           # Lq = 65
RAGGED_F32 = si.Workload("block_ragged_f32", 2, 128, 12, 7, 3, 2, groups=16, dtype="f32",
                         sigma=0.05, seed=5203)
ONE_PATCH = si.Workload("block_n1", 1, 128, 8, 9, 1, 2, seed=5204)            # n = 1: no stale context
ASYNC_CASES = [(W["tiny"], 1), (MID, 2), (RAGGED, 3), (RAGGED_F32, 0), (W["sdxl1024_l2"], 5),
               (ONE_PATCH, 0)]


def _ids(cases):
    return [f"{wl.name}-p{i}" for wl, i in cases]


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("wl,patch", [(W["tiny"], 0), (W["sdxl1024_l2"], 6), (RAGGED, 2)],
                         ids=_ids([(W["tiny"], 0), (W["sdxl1024_l2"], 6), (RAGGED, 2)]))
def test_groupnorm_silu_and_moments(wl, patch):
    wl = wl.with_patch(patch)
    d = cpu_inputs(wl)
    g = gpu_copy(d)
    y, fm = dp.distri_async_groupnorm_silu(wl.geom, wl.groups, g["x_fresh"], g["table"], g["gamma"],
                                           g["beta"], eps=wl.eps)
    z, ref_fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                       d["table"].double().numpy(), d["gamma"], d["beta"])
    assert_close(to_np(y), oracle.silu(z), wl.dtype, f"groupnorm+silu {wl.name}")
    np.testing.assert_allclose(to_np(fm), ref_fm, rtol=1e-5, atol=1e-7)
    # moments straight into the table: slot i = the fresh moments (same bits),
    # every other slot untouched
    tab = g["table"].clone()
    dp.distri_group_moments(wl.geom, wl.groups, g["x_fresh"], tab)
    _, fm2 = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"])
    tb, ob = _bits(tab), _bits(g["table"])
    assert torch.equal(tb[:, patch], _bits(fm2))
    keep = [j for j in range(wl.n_patches) if j != patch]
    assert torch.equal(tb[:, keep], ob[:, keep])


def _block_inputs(wl):
    d = si.make_block_inputs(wl)
    wts = dict(si.block_scalars(wl))
    wts.update({k: v.double().numpy() for k, v in d["weights"].items()})
    return d, wts


def _gpu_state(st):
    return {k: v.cuda().clone() for k, v in st.items()}


def _run_block(wl, d, x, st_in, st_out=None):
    gw = {k: v.cuda() for k, v in d["weights"].items()}
    return dp.distri_patch_block(wl.geom, gw, x, st_in, st_out, groups=wl.groups, heads=wl.heads,
                                 eps=wl.eps, scale=wl.head_dim ** -0.5)


def _check_moments(got, ref, eps, what):
    """Raw group moments (m1, m2) against the oracle's.  gn1 is taken over the
    block input, the same values on both sides: only fp32 summation error,
    eps = 1e-5.  gn2 is taken over the conv output, which the GPU holds in the
    activation dtype: if every value is within eps * RMS of the exact one
    (the parity bound), then |d m1| <= eps * RMS and |d m2| <= (2 eps +
    eps^2) RMS^2, with RMS^2 = m2 of the group."""
    m2 = np.abs(ref[..., 1])
    assert np.all(np.abs(got[..., 0] - ref[..., 0]) <= eps * np.sqrt(m2) + 1e-7), what
    assert np.all(np.abs(got[..., 1] - ref[..., 1]) <= (2 * eps + eps * eps) * m2 + 1e-7), what


def _compare_state(wl, got, ref, before, what):
    """Patch i's rows / slots against the oracle; all else bitwise as before."""
    i, h, Lq, n = wl.patch, wl.h, wl.lq, wl.n_patches
    for key, sl in (("conv_in", slice(i * h, (i + 1) * h)), ("k", slice(i * Lq, (i + 1) * Lq)),
                    ("v", slice(i * Lq, (i + 1) * Lq))):
        assert_close(to_np(got[key][:, sl]), ref[key][:, sl], wl.dtype, f"{what} state {key}")
        keep = torch.ones(got[key].shape[1], dtype=torch.bool)
        keep[sl] = False
        assert torch.equal(_bits(got[key])[:, keep], _bits(before[key])[:, keep]), f"{what} {key}"
    for key in ("gn1", "gn2"):
        _check_moments(to_np(got[key][:, i]), ref[key][:, i], 1e-5 if key == "gn1" else TOL[wl.dtype],
                       f"{what} {key}")
        keep = [j for j in range(n) if j != i]
        assert torch.equal(_bits(got[key])[:, keep], _bits(before[key])[:, keep]), f"{what} {key}"


@pytest.mark.parametrize("wl,patch", ASYNC_CASES, ids=_ids(ASYNC_CASES))
def test_block_async_step(wl, patch):
    wl = wl.with_patch(patch)
    d, wts = _block_inputs(wl)
    h = wl.h
    x_cpu = d["x"][:, patch * h:(patch + 1) * h].contiguous()
    x = x_cpu.cuda()
    st_in = _gpu_state(d["state"])
    st_out = _gpu_state(d["state"])
    y = _run_block(wl, d, x, st_in, st_out)
    ref_y, ref_st = oracle.patch_block(wl.geom, wts, x_cpu, d["state"], act_dtype=wl.dtype)
    tag = f"block {wl.name} patch {patch}"
    assert_close(to_np(y), ref_y, wl.dtype, tag)
    _compare_state(wl, st_out, ref_st, d["state"], tag)
    for k in st_in:                     # state_in is only read
        assert torch.equal(_bits(st_in[k]), _bits(d["state"][k])), k
    # in place (state_out = state_in): the same bits everywhere
    st_same = _gpu_state(d["state"])
    y2 = _run_block(wl, d, x, st_same)
    assert torch.equal(_bits(y2), _bits(y))
    for k in st_same:
        assert torch.equal(_bits(st_same[k]), _bits(st_out[k])), k


@pytest.mark.parametrize("wl", [MID, W["tiny"], RAGGED_F32], ids=["block_mid", "tiny", "ragged_f32"])
def test_block_warmup_then_async_step(wl):
    """Step 1 synchronous over all patches on the previous map, step 2
    asynchronous for patch i on the current map, against the oracle's own two
    steps."""
    wl = wl.with_patch(wl.n_patches - 2)
    d, wts = _block_inputs(wl)
    B, H, Wd, C, n, h, Lq = wl.batch, wl.height, wl.width, wl.channels, wl.n_patches, wl.h, wl.lq
    xp = d["x_prev"]
    xp_patches = xp.view(B, n, h, Wd, C).transpose(0, 1).contiguous().cuda()  # [n, B, h, W, C]
    st = _gpu_state(d["state"])            # contents are overwritten by the sync step
    y_sync = dp.distri_patch_block_sync(wl.geom, {k: v.cuda() for k, v in d["weights"].items()},
                                        xp_patches, st, groups=wl.groups, heads=wl.heads, eps=wl.eps,
                                        scale=wl.head_dim ** -0.5)
    ref_sync, ref_st = oracle.patch_block_sync(wl.geom, wts, xp, act_dtype=wl.dtype)
    got = to_np(y_sync).transpose(1, 0, 2, 3).reshape(B, n * Lq, C)
    assert_close(got, ref_sync, wl.dtype, f"block sync {wl.name}")
    for key in ("conv_in", "k", "v"):
        assert_close(to_np(st[key]), ref_st[key], wl.dtype, f"block sync state {key}")
    _check_moments(to_np(st["gn1"]), ref_st["gn1"], 1e-5, "block sync gn1")
    _check_moments(to_np(st["gn2"]), ref_st["gn2"], TOL[wl.dtype], "block sync gn2")

    i = wl.patch
    x_cpu = d["x"][:, i * h:(i + 1) * h].contiguous()
    y = _run_block(wl, d, x_cpu.cuda(), st)
    # step 2 reads the state as the library holds it: maps in the activation
    # dtype, moment tables in fp32
    held = {k: oracle.round_to(v, wl.dtype if k in ("conv_in", "k", "v") else "f32")
            for k, v in ref_st.items()}
    ref_y, _ = oracle.patch_block(wl.geom, wts, x_cpu, held, act_dtype=wl.dtype)
    assert_close(to_np(y), ref_y, wl.dtype, f"block step 2 {wl.name}")


def test_block_equals_its_ops_at_full_size():
    """At the 3840^2 level-2 shapes the block is bit for bit the chain of the
    single-op calls (same kernels, same launches), and finite."""
    wl = W["sdxl3840_l2"].with_patch(4)
    d = si.make_block_inputs(wl, device="cuda")
    gw = d["weights"]
    B, H, Wd, C, n, h, Lq, L = (wl.batch, wl.height, wl.width, wl.channels, wl.n_patches, wl.h,
                                wl.lq, wl.tokens)
    i = wl.patch
    x = d["x"][:, i * h:(i + 1) * h].contiguous()
    st = {k: v.clone() for k, v in d["state"].items()}
    y = dp.distri_patch_block(wl.geom, gw, x, d["state"], st, groups=wl.groups, heads=wl.heads,
                              eps=wl.eps, scale=0.125)
    s0 = d["state"]
    g1, fm1 = dp.distri_async_groupnorm_silu(wl.geom, wl.groups, x, s0["gn1"], gw["gn1_gamma"],
                                             gw["gn1_beta"], eps=wl.eps)
    hh = dp.distri_patch_conv3x3_halo(wl.geom, g1, s0["conv_in"], gw["conv_w"], gw["conv_b"])
    n2, fm2 = dp.distri_async_groupnorm(wl.geom, wl.groups, hh, s0["gn2"], gw["gn2_gamma"],
                                        gw["gn2_beta"], eps=wl.eps)
    ks, vs = s0["k"].clone(), s0["v"].clone()
    q, k, v = dp.distri_patch_qkv_proj(wl.geom, n2.view(B, Lq, C), gw["w_qkv"], gw["b_qkv"],
                                       k_stale=ks, v_stale=vs)
    o = dp.distri_patch_self_attn(wl.geom, wl.heads, q.view(B, Lq, wl.heads, 64),
                                  k.view(B, Lq, wl.heads, 64), v.view(B, Lq, wl.heads, 64),
                                  s0["k"].view(B, L, wl.heads, 64), s0["v"].view(B, L, wl.heads, 64),
                                  scale=0.125)
    y_ref = dp.distri_patch_out_proj(wl.geom, o.view(B, Lq, C), gw["w_o"], gw["b_o"])
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    assert torch.equal(_bits(y), _bits(y_ref))
    assert torch.equal(_bits(st["k"]), _bits(ks)) and torch.equal(_bits(st["v"]), _bits(vs))
    assert torch.equal(_bits(st["conv_in"][:, i * h:(i + 1) * h]), _bits(g1))
    assert torch.equal(_bits(st["gn1"][:, i]), _bits(fm1))
    assert torch.equal(_bits(st["gn2"][:, i]), _bits(fm2))
