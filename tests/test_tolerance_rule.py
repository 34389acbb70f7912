"""The parity rule max|y - x| <= tol * RMS(x), checked on the CPU.

A bf16 output that is the exact result rounded once (RNE) must pass it on
the attention workload with the heaviest tails, so the bound is one a bf16
kernel can meet; a result perturbed by 2.5e-2 x RMS at a single element, or
one whose rounding of the weights costs a few bf16 ulps, must fail it.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tests.parity_util import TOL, assert_close, rel_max_err


@pytest.fixture(scope="module")
def attn_ref():
    wl = si.WORKLOADS["sdxl1024_l3"].with_patch(1)
    d = si.make_inputs(wl, nonzero_bias=True)
    return oracle.patch_self_attn(wl.geom, wl.heads, 64, 0.125, d["q"], d["k_fresh"], d["v_fresh"],
                                  d["k_stale"], d["v_stale"])


def test_correctly_rounded_bf16_output_passes(attn_ref):
    rounded = torch.from_numpy(attn_ref).to(torch.bfloat16).double().numpy()
    e = assert_close(rounded, attn_ref, "bf16", "oracle rounded to bf16")
    # the rounding alone spends most of the budget on these heavy tails
    assert 0.012 < e < TOL["bf16"]


def test_one_perturbed_element_fails(attn_ref):
    rms = float(np.sqrt(np.mean(attn_ref ** 2)))
    bad = attn_ref.copy()
    bad.flat[12345] += 2.5e-2 * rms
    with pytest.raises(AssertionError):
        assert_close(bad, attn_ref, "bf16", "planted error")
    fine = attn_ref.copy()
    fine.flat[12345] += 1.5e-2 * rms
    assert assert_close(fine, attn_ref, "bf16", "error inside the bound") == pytest.approx(1.5e-2)


def test_fp32_bound_is_relative_to_rms():
    x = np.linspace(-3, 3, 1001)
    rms = float(np.sqrt(np.mean(x * x)))
    assert rel_max_err(x + 0.5e-4 * rms, x) == pytest.approx(0.5e-4)
    assert_close(x + 0.9e-4 * rms, x, "f32", "fp32 inside")
    with pytest.raises(AssertionError):
        assert_close(x + 1.1e-4 * rms, x, "f32", "fp32 outside")


def test_round_to_matches_single_rounding_and_breaks_ties_to_even():
    """oracle.round_to pinned to torch's binary32 -> bf16 conversion (one
    rounding, RNE) on values that binary32 holds exactly, to hand-made ties,
    and to a value just above a midpoint that a detour through binary32
    would round twice, the wrong way."""
    import oracle

    gen = torch.Generator().manual_seed(11)
    x32 = torch.randn(100000, generator=gen) * torch.exp(4 * torch.randn(100000, generator=gen))
    want = x32.to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_to(x32.double().numpy(), "bf16"), want)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(2 + 2.0 ** -7), 0.0])
    np.testing.assert_array_equal(oracle.round_to(ties, "bf16"), [1.0, 1 + 2.0 ** -6, -2.0, 0.0])
    above = 1 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_to(np.array([above]), "bf16")[0] == 1 + 2.0 ** -7
    assert torch.tensor([above], dtype=torch.float64).to(torch.bfloat16).item() == 1.0
    x64 = np.random.default_rng(3).standard_normal(1000)
    np.testing.assert_array_equal(oracle.round_to(x64, "f32"), x64.astype(np.float32).astype(np.float64))


def test_where_the_floor_exceeds_the_bound_elements_must_be_correctly_rounded():
    """A SiLU-shaped heavy tail: rounding alone exceeds 2e-2 x RMS.  The
    correctly rounded output passes; the other neighbour of an element that
    is not near a midpoint fails."""
    import oracle
    from tests.parity_util import rounding_floor

    z = np.random.default_rng(5).standard_normal(200000)
    x = z / (1 + np.exp(-z))
    assert rounding_floor(x, "bf16") > TOL["bf16"]
    assert_close(oracle.round_to(x, "bf16"), x, "bf16", "silu rounded")
    bad = oracle.round_to(x, "bf16")
    k = int(np.argmax(np.abs(x)))
    step = 2.0 ** (np.frexp(abs(x[k]))[1] - 8)
    bad[k] += step if bad[k] < x[k] else -step    # the other neighbour
    if abs(abs(bad[k] - x[k]) - step / 2) > 2.0 ** -12 * abs(x[k]):
        with pytest.raises(AssertionError):
            assert_close(bad, x, "bf16", "silu wrong neighbour")
