"""Kernels at the size limits the ABI accepts, checked through closed forms
that hold at any size (the oracle cannot walk multi-GB maps).

 * Attention at H*W*heads*64 just below 2^31 (the 32-bit offset bound):
   with every key equal, the softmax is uniform, so every query row returns
   the mean of the hybrid V over all tokens.
 * Conv at B*H*W*Cin just below 2^31: a weight whose only non-zero tap is
   (kh, kw) = (0, 0) with the identity over channels makes y[r, c] the input
   pixel (r-1, c-1) of the hybrid map - the stale halo row above the patch,
   zero in column 0 - plus the bias, rounded once.
 * Refresh of the same multi-GB map: the patch rows change bitwise, the
   rest not at all.
"""
import pytest
import torch

import displaced_patch_parallelism_distri_amd as dp

pytestmark = pytest.mark.gpu

H = W = 1824          # H*W*640 = 2_129_264_640 < 2^31
N_PATCH = 96          # h = 19 rows, Lq = 34656
PATCH = 50
HEADS, D = 10, 64
C = HEADS * D


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()
    assert H * W * C < 2 ** 31


def _randn_bf16(shape, gen, mean=0.0):
    return (torch.randn(shape, generator=gen, device="cuda") + mean).to(torch.bfloat16)


def test_attention_at_the_offset_limit_uniform_keys():
    gen = torch.Generator(device="cuda").manual_seed(5150)
    h = H // N_PATCH
    lq, L = h * W, H * W
    geom = (1, H, W, N_PATCH, PATCH)
    q = _randn_bf16((1, lq, HEADS, D), gen)
    kvec = _randn_bf16((1, 1, HEADS, D), gen)
    k_fresh = kvec.expand(1, lq, HEADS, D).contiguous()
    k_stale = kvec.expand(1, L, HEADS, D).contiguous()
    v_fresh = _randn_bf16((1, lq, HEADS, D), gen, mean=0.5)
    v_stale = _randn_bf16((1, L, HEADS, D), gen, mean=0.5)
    out = dp.distri_patch_self_attn(geom, HEADS, q, k_fresh, v_fresh, k_stale, v_stale)
    torch.cuda.synchronize()
    lo = PATCH * lq
    total = v_stale[0].double().sum(0) - v_stale[0, lo:lo + lq].double().sum(0) + v_fresh[0].double().sum(0)
    mean = (total / L).float()                                   # [heads, d]
    want = mean.to(torch.bfloat16).float()
    got = out[0].float()                                         # [lq, heads, d]
    # every row equals the bf16-rounded mean to within one bf16 ulp
    ulp = torch.ldexp(torch.ones_like(want), torch.frexp(want.abs())[1] - 8)
    assert torch.all((got - want).abs() <= ulp), float(((got - want).abs() / ulp).max())
    del k_stale, v_stale


def test_conv_and_refresh_at_the_offset_limit():
    gen = torch.Generator(device="cuda").manual_seed(5151)
    h = H // N_PATCH
    geom = (1, H, W, N_PATCH, PATCH)
    x_fresh = _randn_bf16((1, h, W, C), gen)
    x_stale = _randn_bf16((1, H, W, C), gen)
    weight = torch.zeros(C, 3, 3, C, dtype=torch.bfloat16, device="cuda")
    weight[:, 0, 0, :] = torch.eye(C, dtype=torch.bfloat16, device="cuda")
    bias = torch.randn(C, generator=gen, device="cuda") * 0.25
    y = dp.distri_patch_conv3x3_halo(geom, x_fresh, x_stale, weight, bias)
    torch.cuda.synchronize()
    # hybrid input rows r-1 for r = 0..h-1: the stale halo row, then fresh rows
    src = torch.cat([x_stale[:, PATCH * h - 1:PATCH * h], x_fresh[:, :h - 1]], dim=1)
    shifted = torch.zeros_like(src)
    shifted[:, :, 1:] = src[:, :, :-1]                           # column c-1, zero at c = 0
    want = (shifted.float() + bias).to(torch.bfloat16)
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))

    # refresh the same map: patch rows take the fresh slice, others unchanged
    before_top = x_stale[:, PATCH * h - 1].clone()
    before_bottom = x_stale[:, (PATCH + 1) * h].clone()
    dp.distri_refresh_stale(geom, W * C, x_fresh, x_stale)
    torch.cuda.synchronize()
    assert torch.equal(x_stale[:, PATCH * h:(PATCH + 1) * h].view(torch.int16), x_fresh.view(torch.int16))
    assert torch.equal(x_stale[:, PATCH * h - 1].view(torch.int16), before_top.view(torch.int16))
    assert torch.equal(x_stale[:, (PATCH + 1) * h].view(torch.int16), before_bottom.view(torch.int16))
