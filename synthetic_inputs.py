"""Seeded synthetic inputs for the patch-layer workloads.

This module only draws random numbers and slices them; it holds none of the
method's arithmetic, so the oracle side and the HIP side can both take their
inputs from it.

Workloads are SDXL UNet feature maps at the shapes of the 1024^2, 2048^2 and
3840^2 latents (SDXL compresses images 8x into its latent space: "阅读论文1_d-
CSDN博客", section 实验设置, 模型), split by rows into n patches.  The real
benchmark uses SDXL weights and COCO captions, neither of which is used here:
seeded N(0,1) activations stand in for them.

Recipe (per workload, torch generator seeded with ``seed``), drawn in this
order on the chosen device:
  1. X_full  [B, H, W, C]          ~ N(0, 1)
  2. noise_x [B, H, W, C]          ~ N(0, 1)
  3. Q_full, K_full, V_full  [B, H*W, heads, d]  ~ N(0, 1)
  4. noise_k, noise_v        [B, H*W, heads, d]  ~ N(0, 1)
  5. conv weight [C, 3, 3, C]      ~ N(0, 1 / (9 C))
  6. gamma = 1 + 0.1 N(0,1), beta = 0.1 N(0,1)   [C], fp32
  7. conv bias [C] = 0, or 0.1 N(0,1) with ``nonzero_bias``
stale maps = full + sigma * noise (or exactly full with ``stale_equals_fresh``);
fresh tensors are the rows / tokens of patch i of the full maps.  Values are
rounded (round-to-nearest-even) to the workload dtype after the stale sum.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    channels: int
    height: int
    width: int
    n_patches: int
    heads: int
    head_dim: int = 64
    groups: int = 32
    eps: float = 1e-5
    dtype: str = "bf16"
    sigma: float = 0.1
    seed: int = 1000
    patch: int = 0

    @property
    def geom(self):
        return (self.batch, self.height, self.width, self.n_patches, self.patch)

    @property
    def h(self):
        return self.height // self.n_patches

    @property
    def lq(self):
        return self.h * self.width

    @property
    def tokens(self):
        return self.height * self.width

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_patch(self, i):
        return replace(self, patch=i)

    # algorithmic work: attention counts Q K^T and P V (not the softmax); the
    # conv counts all 9 taps, zero-padded edge taps included
    def attn_flops(self):
        return 4.0 * self.batch * self.heads * self.lq * self.tokens * self.head_dim

    def conv_flops(self):
        return 2.0 * self.batch * self.lq * self.channels * self.channels * 9

    def elem_bytes(self):
        return 4 if self.dtype == "f32" else 2

    def slice_bytes(self):
        """Bytes of one fresh slice [B, h, W, C]."""
        return self.batch * self.lq * self.channels * self.elem_bytes()


WORKLOADS = {
    "tiny": Workload("tiny", 1, 128, 32, 32, 2, 2, dtype="f32", sigma=0.05, seed=1001),
    "sdxl1024_l2": Workload("sdxl1024_l2", 2, 640, 64, 64, 8, 10, seed=1002),
    "sdxl1024_l3": Workload("sdxl1024_l3", 2, 1280, 32, 32, 4, 20, seed=1003),
    "sdxl2048_l2": Workload("sdxl2048_l2", 2, 640, 128, 128, 8, 10, seed=1004),
    "sdxl3840_l2": Workload("sdxl3840_l2", 2, 640, 240, 240, 8, 10, seed=1005),
    "sdxl3840_l3": Workload("sdxl3840_l3", 2, 1280, 120, 120, 8, 20, seed=1006),
}


def make_inputs(wl: Workload, device="cpu", stale_equals_fresh=False, nonzero_bias=False):
    """Draw the seeded tensors of ``wl`` and cut out patch ``wl.patch``.

    Returns a dict of contiguous tensors on ``device`` in the workload dtype
    (gamma, beta, bias in fp32)."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed)
    B, H, W, C = wl.batch, wl.height, wl.width, wl.channels
    L, nh, d = wl.tokens, wl.heads, wl.head_dim
    h, i, Lq = wl.h, wl.patch, wl.lq
    dt = wl.torch_dtype

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    x_full = randn(B, H, W, C)
    noise_x = randn(B, H, W, C)
    q_full = randn(B, L, nh, d)
    k_full = randn(B, L, nh, d)
    v_full = randn(B, L, nh, d)
    noise_k = randn(B, L, nh, d)
    noise_v = randn(B, L, nh, d)
    weight = randn(C, 3, 3, C) * (1.0 / (9.0 * C)) ** 0.5
    gamma = 1.0 + 0.1 * randn(C)
    beta = 0.1 * randn(C)
    bias = 0.1 * randn(C) if nonzero_bias else torch.zeros(C, device=device)

    s = 0.0 if stale_equals_fresh else wl.sigma
    x_stale = (x_full + s * noise_x).to(dt)
    k_stale = (k_full + s * noise_k).to(dt)
    v_stale = (v_full + s * noise_v).to(dt)
    del noise_x, noise_k, noise_v
    out = {
        "x_fresh": x_full[:, i * h:(i + 1) * h].to(dt).contiguous(),
        "x_stale": x_stale.contiguous(),
        "q": q_full[:, i * Lq:(i + 1) * Lq].to(dt).contiguous(),
        "k_fresh": k_full[:, i * Lq:(i + 1) * Lq].to(dt).contiguous(),
        "v_fresh": v_full[:, i * Lq:(i + 1) * Lq].to(dt).contiguous(),
        "k_stale": k_stale.contiguous(),
        "v_stale": v_stale.contiguous(),
        "weight": weight.to(dt).contiguous(),
        "bias": bias.contiguous(),
        "gamma": gamma.contiguous(),
        "beta": beta.contiguous(),
    }
    return out


def make_map(shape, seed, dtype=torch.float32, device="cpu", scale=1.0):
    """A single seeded N(0, scale^2) tensor, rounded to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g, device=device, dtype=torch.float32)).to(dtype)


def make_proj_inputs(wl: Workload, device="cpu"):
    """Seeded inputs of the attention layer's projections for patch
    ``wl.patch`` (their own generator, seeded with ``seed + 7919``, so the
    tensors of ``make_inputs`` are unchanged).  Drawn in this order:
      1. x      [B, Lq, C]   ~ N(0, 1)     hidden states of the patch's tokens
      2. w_qkv  [3C, C]      ~ N(0, 1 / C) Q, K, V weights stacked by rows
      3. b_qkv  [3C] fp32    = 0.1 N(0, 1)
      4. o      [B, Lq, C]   ~ N(0, 1)     attention output of the patch
      5. w_o    [C, C]       ~ N(0, 1 / C)
      6. b_o    [C] fp32     = 0.1 N(0, 1)
      7. k_stale, v_stale [B, H*W, C] ~ N(0, 1)  last step's K / V maps
    Rounded to the workload dtype (biases stay fp32)."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed + 7919)
    B, C, L, Lq = wl.batch, wl.channels, wl.tokens, wl.lq
    dt = wl.torch_dtype

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    out = {
        "x": randn(B, Lq, C).to(dt),
        "w_qkv": (randn(3 * C, C) * C ** -0.5).to(dt),
        "b_qkv": 0.1 * randn(3 * C),
        "o": randn(B, Lq, C).to(dt),
        "w_o": (randn(C, C) * C ** -0.5).to(dt),
        "b_o": 0.1 * randn(C),
    }
    out["k_stale"] = randn(B, L, C).to(dt)
    out["v_stale"] = randn(B, L, C).to(dt)
    return {k: v.contiguous() for k, v in out.items()}


def make_block_inputs(wl: Workload, device="cpu"):
    """Seeded inputs of the patch block (GroupNorm + SiLU -> conv ->
    GroupNorm -> Q/K/V projection -> attention -> output projection) at the
    shapes of ``wl`` (C = heads * head_dim); own generator, seeded with
    ``seed + 104729``.  Drawn in this order:
      1. x      [B, H, W, C]  ~ N(0, 1)    this step's full input map
      2. x_prev [B, H, W, C]  = x + sigma N(0, 1)   the previous step's
      3. conv_w [C, 3, 3, C]  ~ N(0, 1 / (9 C)),  conv_b = 0.1 N(0, 1)
      4. gn1_gamma = 1 + 0.1 N, gn1_beta = 0.1 N, then gn2_gamma, gn2_beta
      5. w_qkv [3C, C] ~ N(0, 1 / C), b_qkv = 0.1 N;  w_o [C, C], b_o likewise
      6. a random previous-step state: conv_in [B, H, W, C] ~ N(0, 1);
         k, v [B, H*W, C] ~ N(0, 1); moment tables gn1, gn2 [B, n, G, 2]
         with first moment 0.1 N(0, 1) and second moment first^2 + U(0.5, 1.5)
    Tensors in the workload dtype; biases, gammas, betas and tables fp32."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed + 104729)
    B, H, W, C, n, G = wl.batch, wl.height, wl.width, wl.channels, wl.n_patches, wl.groups
    L = H * W
    dt = wl.torch_dtype

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    def table():
        m1 = 0.1 * randn(B, n, G)
        m2 = m1 * m1 + 0.5 + torch.rand(B, n, G, generator=g, device=device)
        return torch.stack([m1, m2], dim=-1).contiguous()

    x = randn(B, H, W, C)
    x_prev = x + wl.sigma * randn(B, H, W, C)
    wts = {
        "conv_w": (randn(C, 3, 3, C) * (1.0 / (9.0 * C)) ** 0.5).to(dt),
        "conv_b": 0.1 * randn(C),
        "gn1_gamma": 1.0 + 0.1 * randn(C),
        "gn1_beta": 0.1 * randn(C),
        "gn2_gamma": 1.0 + 0.1 * randn(C),
        "gn2_beta": 0.1 * randn(C),
        "w_qkv": (randn(3 * C, C) * C ** -0.5).to(dt),
        "b_qkv": 0.1 * randn(3 * C),
        "w_o": (randn(C, C) * C ** -0.5).to(dt),
        "b_o": 0.1 * randn(C),
    }
    state = {
        "conv_in": randn(B, H, W, C).to(dt),
        "k": randn(B, L, C).to(dt),
        "v": randn(B, L, C).to(dt),
        "gn1": table(),
        "gn2": table(),
    }
    out = {"x": x.to(dt), "x_prev": x_prev.to(dt), "weights": wts, "state": state}
    for d in (wts, state):
        for k in d:
            d[k] = d[k].contiguous()
    return out


def block_scalars(wl: Workload):
    """The block's non-tensor parameters at the shapes of ``wl``."""
    return {"channels": wl.channels, "groups": wl.groups, "heads": wl.heads, "eps": wl.eps,
            "scale": wl.head_dim ** -0.5}


def make_cross_inputs(wl: Workload, ctx_len=77, device="cpu"):
    """Seeded inputs of cross-attention with patch queries (own generator,
    seeded with ``seed + 15485863``): q [B, Lq, heads, d] then k_ctx, v_ctx
    [B, ctx_len, heads, d], all ~ N(0, 1), in the workload dtype.  77 is the
    token count of SDXL's text encoders."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed + 15485863)
    B, nh, d = wl.batch, wl.heads, wl.head_dim
    dt = wl.torch_dtype

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(dt).contiguous()

    return {"q": randn(B, wl.lq, nh, d), "k_ctx": randn(B, ctx_len, nh, d),
            "v_ctx": randn(B, ctx_len, nh, d)}
