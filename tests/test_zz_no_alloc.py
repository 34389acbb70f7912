"""The allocation-free GroupNorm entry point, through the C ABI, against the
workspace form on the same inputs: bit for bit (the same kernels run), and
within the parity bound of the oracle, on two calls in a row, the second on
a smaller input (the scratch keeps the first call's contents), for bf16 and
fp32.
"""
import ctypes

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


def _noalloc(wl, g, y, fm):
    lib = dp.load()
    code = dp.DISTRI_BF16 if wl.dtype == "bf16" else dp.DISTRI_F32
    st = lib.distri_async_groupnorm_noalloc(
        ctypes.byref(dp.geom(*wl.geom)), wl.channels, wl.groups, wl.eps, code,
        g["x_fresh"].data_ptr(), g["table"].data_ptr(), g["gamma"].data_ptr(), g["beta"].data_ptr(),
        y.data_ptr(), fm.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.distri_last_error()


def _bits(t):
    return t.detach().cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("first,second", [(("sdxl3840_l2", 4), ("sdxl1024_l3", 1)),
                                          (("sdxl1024_l2", 6), ("tiny", 0))],
                         ids=["3840_then_1024", "1024_then_fp32_tiny"])
def test_noalloc_groupnorm_matches_the_workspace_form(first, second):
    for name, patch in (first, second):
        wl = si.WORKLOADS[name].with_patch(patch)
        d = cpu_inputs(wl)
        g = gpu_copy(d)
        y_ws, fm_ws = dp.distri_async_groupnorm(wl.geom, wl.groups, g["x_fresh"], g["table"],
                                                g["gamma"], g["beta"], eps=wl.eps)
        y = torch.full_like(g["x_fresh"], float("nan"))
        fm = torch.full((wl.batch, wl.groups, 2), float("nan"), device="cuda")
        _noalloc(wl, g, y, fm)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ws)), f"{name}: y differs from the workspace form"
        assert torch.equal(_bits(fm), _bits(fm_ws)), f"{name}: moments differ"
        ref_y, ref_fm = oracle.async_groupnorm(wl.geom, wl.channels, wl.groups, wl.eps, d["x_fresh"],
                                               d["table"].double().numpy(), d["gamma"], d["beta"])
        assert_close(to_np(y), ref_y, wl.dtype, f"groupnorm noalloc {name} patch {patch}")
        np.testing.assert_allclose(to_np(fm), ref_fm, rtol=1e-5, atol=1e-7)
