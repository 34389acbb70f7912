"""Pins of the oracle's patch block (a chain of the oracle's layer routines)
against checks that do not reuse it:

* with n = 1 the block is the plain full-image block, computed here with
  torch's own fp64 library layers (group_norm, silu, conv2d, linear, softmax);
* the synchronous step over all patches reproduces the n = 1 block on the same
  map, row for row (the method's claim that the warm-up step with all current
  activations is exact);
* an asynchronous step whose stale state is the synchronous step's own
  state on the same input (stale = fresh) gives the same rows again;
* the asynchronous step changes only patch i's rows / slots of the state, and
  those hold its own fresh values;
* with act_dtype = "bf16" (every op fed bf16 tensors) the n = 1 block and the
  synchronous step equal torch's fp64 library block with the same tensors
  rounded to bf16 by a bit-level round-to-nearest-even written here.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.filterwarnings("ignore")

SMALL = si.Workload("block_small", 2, 128, 8, 6, 4, 2, groups=8, dtype="f32", seed=5101)


def _wts(wl, d):
    w = dict(si.block_scalars(wl))
    w.update({k: v.double().numpy() for k, v in d["weights"].items()})
    return w


def _state(d):
    return {k: v.double().numpy() for k, v in d["state"].items()}


def _bits_rne_bf16(a):
    """float64 tensor -> nearest bf16 value (8 significant bits), ties to
    even, by integer arithmetic on the binary64 encoding: drop the low 45 of
    its 52 fraction bits after adding half of that unit (minus one, plus the
    lowest kept bit, which breaks ties to even)."""
    b = a.contiguous().view(torch.int64)
    keep = (b >> 45) & 1
    b = (b + ((1 << 44) - 1) + keep) & ~((1 << 45) - 1)
    return b.view(torch.float64)


def _torch_block(wl, w, x, rnd=lambda a: a):
    """Full-image block with torch fp64 library layers; x [B, H, W, C].
    ``rnd`` is applied to each layer's result that the next layer reads."""
    B, H, W, C = x.shape
    nh, d = wl.heads, C // wl.heads
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    xc = t(x).permute(0, 3, 1, 2)
    z = rnd(F.silu(F.group_norm(xc, wl.groups, t(w["gn1_gamma"]), t(w["gn1_beta"]), wl.eps)))
    wc = t(w["conv_w"]).permute(0, 3, 1, 2)  # [Cout, Cin, 3, 3]
    hh = rnd(F.conv2d(z, wc, t(w["conv_b"]), padding=1))
    n2 = rnd(F.group_norm(hh, wl.groups, t(w["gn2_gamma"]), t(w["gn2_beta"]), wl.eps))
    tok = n2.permute(0, 2, 3, 1).reshape(B, H * W, C)
    qkv = rnd(F.linear(tok, t(w["w_qkv"]), t(w["b_qkv"])))
    q, k, v = (a.reshape(B, H * W, nh, d).transpose(1, 2) for a in qkv.split(C, dim=-1))
    p = torch.softmax(q @ k.transpose(-1, -2) * w["scale"], dim=-1)
    o = rnd((p @ v).transpose(1, 2).reshape(B, H * W, C))
    return F.linear(o, t(w["w_o"]), t(w["b_o"])).numpy()


def test_single_patch_block_is_the_library_block():
    wl = SMALL
    full = si.Workload(wl.name, wl.batch, wl.channels, wl.height, wl.width, 1, wl.heads,
                       groups=wl.groups, dtype="f32", seed=wl.seed)
    d = si.make_block_inputs(full)
    w = _wts(full, d)
    x = d["x"].double().numpy()
    y, _ = oracle.patch_block(full.geom, w, x, _state(d))
    ref = _torch_block(full, w, x)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-10)


def test_bit_rounding_helper():
    x = torch.tensor([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30, -3.1, 0.0],
                     dtype=torch.float64)
    want = [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -3.09375, 0.0]
    assert _bits_rne_bf16(x).tolist() == want
    y = torch.randn(10000, dtype=torch.float32).double()   # binary32 values: one rounding
    assert torch.equal(_bits_rne_bf16(y), y.float().to(torch.bfloat16).double())


def test_block_with_bf16_tensors_is_the_rounded_library_block():
    wl = SMALL
    full = si.Workload(wl.name, wl.batch, wl.channels, wl.height, wl.width, 1, wl.heads,
                       groups=wl.groups, dtype="f32", seed=wl.seed)
    d = si.make_block_inputs(full)
    w = _wts(full, d)
    x = d["x"].double().numpy()
    ref = _torch_block(full, w, x, _bits_rne_bf16)
    y, _ = oracle.patch_block(full.geom, w, x, _state(d), act_dtype="bf16")
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-10)
    assert not np.allclose(y, _torch_block(full, w, x), rtol=1e-5, atol=1e-6)
    d4 = si.make_block_inputs(wl)
    y_sync, _ = oracle.patch_block_sync(wl.geom, _wts(wl, d4), d4["x"].double().numpy(),
                                        act_dtype="bf16")
    np.testing.assert_allclose(y_sync, _torch_block(wl, _wts(wl, d4), d4["x"].double().numpy(),
                                                    _bits_rne_bf16), rtol=1e-9, atol=1e-10)


def test_sync_step_reproduces_the_full_image_block():
    wl = SMALL
    d = si.make_block_inputs(wl)
    w = _wts(wl, d)
    x = d["x"].double().numpy()
    y, state = oracle.patch_block_sync(wl.geom, w, x)
    ref = _torch_block(wl, w, x)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-10)
    # the state holds every patch's current values
    B, H, W, C, n, G = wl.batch, wl.height, wl.width, wl.channels, wl.n_patches, wl.groups
    h = H // n
    for j in range(n):
        xs = x[:, j * h:(j + 1) * h]
        np.testing.assert_allclose(state["gn1"][:, j, :, 0],
                                   xs.reshape(B, -1, G, C // G).mean(axis=(1, 3)), rtol=1e-12, atol=1e-14)
    assert state["k"].shape == (B, H * W, C) and state["conv_in"].shape == (B, H, W, C)


@pytest.mark.parametrize("patch", [0, 2, 3])
def test_async_step_on_its_own_sync_state_is_exact(patch):
    wl = SMALL.with_patch(patch)
    d = si.make_block_inputs(wl)
    w = _wts(wl, d)
    x = d["x"].double().numpy()
    y_sync, state = oracle.patch_block_sync(wl.geom, w, x)
    h, Lq = wl.h, wl.lq
    y, new = oracle.patch_block(wl.geom, w, x[:, patch * h:(patch + 1) * h], state)
    np.testing.assert_allclose(y, y_sync[:, patch * Lq:(patch + 1) * Lq], rtol=1e-10, atol=1e-12)
    for key in state:
        np.testing.assert_allclose(new[key], state[key], rtol=1e-10, atol=1e-12)


def test_async_step_touches_only_its_own_rows():
    wl = SMALL.with_patch(1)
    d = si.make_block_inputs(wl)
    w = _wts(wl, d)
    st = _state(d)
    B, H, W, C, n, G = wl.batch, wl.height, wl.width, wl.channels, wl.n_patches, wl.groups
    h, Lq, i = wl.h, wl.lq, wl.patch
    x = d["x"].double().numpy()[:, i * h:(i + 1) * h]
    y, new = oracle.patch_block(wl.geom, w, x, st)
    assert y.shape == (B, Lq, C)
    for key, ax_rows in (("conv_in", slice(i * h, (i + 1) * h)), ("k", slice(i * Lq, (i + 1) * Lq)),
                         ("v", slice(i * Lq, (i + 1) * Lq))):
        keep = np.ones(new[key].shape[1], bool)
        keep[ax_rows] = False
        np.testing.assert_array_equal(new[key][:, keep], st[key][:, keep])
        assert not np.allclose(new[key][:, ax_rows], st[key][:, ax_rows])
    for key in ("gn1", "gn2"):
        keep = np.arange(n) != i
        np.testing.assert_array_equal(new[key][:, keep], st[key][:, keep])
    # slot i of gn1 = this patch's raw moments of x; conv_in rows = SiLU(GN1(x))
    np.testing.assert_allclose(new["gn1"][:, i], oracle.group_moments(x, G), rtol=1e-12, atol=1e-15)
    z, _ = oracle.async_groupnorm(wl.geom, C, G, wl.eps, x, st["gn1"], w["gn1_gamma"], w["gn1_beta"])
    np.testing.assert_allclose(new["conv_in"][:, i * h:(i + 1) * h], z / (1 + np.exp(-z)), rtol=1e-14)


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 1e-8])
    y = oracle.silu(z)
    assert y[0] == 0.0
    np.testing.assert_allclose(y[1], 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)
    np.testing.assert_allclose(y[1] - y[2], 1.0, rtol=1e-15)  # silu(z) - silu(-z) = z
    np.testing.assert_allclose(y[3], 40.0, rtol=1e-15)
    assert abs(y[4]) < 1e-15
    np.testing.assert_allclose(y[5], 0.5e-8, rtol=1e-7)
