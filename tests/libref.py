"""Library references used to pin the oracle (test-only).

Each function builds the hybrid map explicitly (the stale map with patch i's
rows replaced by the fresh rows) and applies a torch float64 CPU library
routine to it: ``F.scaled_dot_product_attention``, ``F.conv2d`` and
``F.group_norm``.  These routines are independent of the oracle's C code.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t64(a):
    if isinstance(a, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return a.detach().to("cpu", torch.float64)


def hybrid_tokens(fresh, stale, geom):
    """[B, L, heads, d] stale map with the tokens of patch i taken from fresh."""
    B, H, W, n, i = geom
    Lq = (H // n) * W
    hyb = _t64(stale).clone()
    hyb[:, i * Lq:(i + 1) * Lq] = _t64(fresh)
    return hyb


def hybrid_rows(fresh, stale, geom):
    """[B, H, W, C] stale map with rows of patch i taken from fresh."""
    B, H, W, n, i = geom
    h = H // n
    hyb = _t64(stale).clone()
    hyb[:, i * h:(i + 1) * h] = _t64(fresh)
    return hyb


def attn_ref(geom, scale, q, k_fresh, v_fresh, k_stale, v_stale, rows=None):
    """Rows of softmax(scale Q Khat^T) Vhat via torch's SDPA (float64)."""
    k = hybrid_tokens(k_fresh, k_stale, geom).permute(0, 2, 1, 3)
    v = hybrid_tokens(v_fresh, v_stale, geom).permute(0, 2, 1, 3)
    qq = _t64(q)
    if rows is not None:
        qq = qq[:, rows[0]:rows[1]]
    out = F.scaled_dot_product_attention(qq.permute(0, 2, 1, 3), k, v, scale=scale)
    return out.permute(0, 2, 1, 3).contiguous().numpy()


def conv_ref(geom, x_fresh, x_stale, weight, bias=None, rows=None):
    """Rows R_i of conv2d(Xhat, w, pad=1) via torch (float64), NHWC out."""
    B, H, W, n, i = geom
    h = H // n
    hyb = hybrid_rows(x_fresh, x_stale, geom).permute(0, 3, 1, 2)
    w = _t64(weight).permute(0, 3, 1, 2)  # [Cout, Cin, 3, 3]
    b = None if bias is None else _t64(bias)
    r0, r1 = rows if rows is not None else (0, h)
    # zero-pad the whole hybrid map, then take the padded rows that output
    # rows [lo, hi) read: padded rows lo .. hi+1
    lo, hi = i * h + r0, i * h + r1
    full = F.pad(hyb, (1, 1, 1, 1))
    y = F.conv2d(full[:, :, lo:hi + 2], w, b)
    return y.permute(0, 2, 3, 1).contiguous().numpy()


def patch_moments(x_map, geom, groups):
    """[B, n, G, 2] raw moments of every patch of a full map [B, H, W, C]
    (numpy mean over the group's values)."""
    B, H, W, n, _i = geom
    h = H // n
    x = _t64(x_map).numpy()
    C = x.shape[-1]
    out = np.zeros((B, n, groups, 2))
    for j in range(n):
        blk = x[:, j * h:(j + 1) * h].reshape(B, h * W, groups, C // groups)
        out[:, j, :, 0] = blk.mean(axis=(1, 3))
        out[:, j, :, 1] = (blk * blk).mean(axis=(1, 3))
    return out


def gn_ref(geom, groups, eps, x_fresh, x_stale, gamma=None, beta=None):
    """Rows R_i of F.group_norm(Xhat) (float64), NHWC out."""
    B, H, W, n, i = geom
    h = H // n
    hyb = hybrid_rows(x_fresh, x_stale, geom).permute(0, 3, 1, 2)
    g = None if gamma is None else _t64(gamma)
    b = None if beta is None else _t64(beta)
    y = F.group_norm(hyb, groups, g, b, eps)
    return y[:, :, i * h:(i + 1) * h].permute(0, 2, 3, 1).contiguous().numpy()
