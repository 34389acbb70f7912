"""CPU oracle for one patch layer of DistriFusion's displaced patch parallelism.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The arithmetic lives
in ``oracle.c`` (plain C, float64, OpenMP over independent outputs); this file
only marshals float64 numpy arrays through ctypes.  It shares no code with the
HIP library and the HIP library never calls it.

Every function takes and returns float64 arrays; callers widen bf16 / fp32
values exactly before the call.  Layouts are the ones the C file documents.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_patch_self_attn.argtypes = [_I] * 7 + [ctypes.c_double] + [_D] * 5 + [_I, _I, _D]
        lib.oracle_patch_conv3x3_halo.argtypes = [_I] * 7 + [_D] * 4 + [_I, _I, _D]
        lib.oracle_group_moments.argtypes = [_I] * 5 + [_D, _D]
        lib.oracle_async_groupnorm.argtypes = [_I] * 7 + [ctypes.c_double] + [_D] * 6
        lib.oracle_refresh_stale.argtypes = [_I] * 5 + [_D, _D]
        lib.oracle_linear.argtypes = [_I] * 3 + [_D] * 4
        lib.oracle_patch_qkv_proj.argtypes = [_I] * 6 + [_D] * 8
        for f in ("oracle_patch_self_attn", "oracle_patch_conv3x3_halo", "oracle_group_moments",
                  "oracle_async_groupnorm", "oracle_refresh_stale", "oracle_linear",
                  "oracle_patch_qkv_proj"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu")
        import torch

        a = a.to(torch.float64).numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid shape arguments")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def patch_self_attn(geom, heads, head_dim, scale, q, k_fresh, v_fresh, k_stale, v_stale,
                    rows=None):
    """Attention of patch ``geom.patch`` over the hybrid K/V map.

    q, k_fresh, v_fresh: [B, Lq, heads, d]; k_stale, v_stale: [B, L, heads, d].
    ``rows`` = (r0, r1) restricts the computed local query rows; the result is
    [B, r1 - r0, heads, d] float64.
    """
    B, H, W, n, i = geom
    Lq = (H // n) * W
    r0, r1 = rows if rows is not None else (0, Lq)
    q, kf, vf, ks, vs = (_f64(t) for t in (q, k_fresh, v_fresh, k_stale, v_stale))
    out = np.zeros((B, r1 - r0, heads, head_dim), dtype=np.float64)
    rc = _load().oracle_patch_self_attn(B, H, W, n, i, heads, head_dim, float(scale),
                                        _p(q), _p(kf), _p(vf), _p(ks), _p(vs), r0, r1, _p(out))
    _check(rc, "patch_self_attn")
    return out


def patch_conv3x3_halo(geom, c_in, c_out, x_fresh, x_stale, weight, bias=None, rows=None):
    """3x3 conv of the hybrid map; x_fresh [B,h,W,Cin], x_stale [B,H,W,Cin],
    weight [Cout,3,3,Cin], bias [Cout] or None. Returns [B, r1-r0, W, Cout]."""
    B, H, W, n, i = geom
    h = H // n
    r0, r1 = rows if rows is not None else (0, h)
    xf, xs, w, b = _f64(x_fresh), _f64(x_stale), _f64(weight), _f64(bias)
    y = np.zeros((B, r1 - r0, W, c_out), dtype=np.float64)
    rc = _load().oracle_patch_conv3x3_halo(B, H, W, n, i, c_in, c_out, _p(xf), _p(xs), _p(w),
                                           _p(b), r0, r1, _p(y))
    _check(rc, "patch_conv3x3_halo")
    return y


def group_moments(x, groups):
    """Raw moments (E[x], E[x^2]) per (batch, group) of a map [B, rows, W, C]."""
    x = _f64(x)
    B, rows, W, C = x.shape
    out = np.zeros((B, groups, 2), dtype=np.float64)
    rc = _load().oracle_group_moments(B, rows, W, C, groups, _p(x), _p(out))
    _check(rc, "group_moments")
    return out


def async_groupnorm(geom, channels, groups, eps, x_fresh, stale_moments, gamma=None, beta=None):
    """Corrected asynchronous GroupNorm; returns (y [B,h,W,C], fresh_moments [B,G,2])."""
    B, H, W, n, i = geom
    h = H // n
    xf, sm, ga, be = _f64(x_fresh), _f64(stale_moments), _f64(gamma), _f64(beta)
    y = np.zeros((B, h, W, channels), dtype=np.float64)
    fm = np.zeros((B, groups, 2), dtype=np.float64)
    rc = _load().oracle_async_groupnorm(B, H, W, n, i, channels, groups, float(eps), _p(xf),
                                        _p(sm), _p(ga), _p(be), _p(y), _p(fm))
    _check(rc, "async_groupnorm")
    return y, fm


def refresh_stale(geom, row_elems, fresh, stale):
    """Returns a copy of ``stale`` [B,H,row_elems] with patch i's rows replaced
    by ``fresh`` [B,h,row_elems]."""
    B, H, _W, n, i = geom
    f = _f64(fresh)
    s = _f64(stale).copy()
    rc = _load().oracle_refresh_stale(B, H, n, i, row_elems, _p(f), _p(s))
    _check(rc, "refresh_stale")
    return s


def linear(x, weight, bias=None):
    """Token-wise linear map: x [..., C], weight [N, C], bias [N] or None ->
    [..., N] float64 (y = x W^T + b)."""
    xf = _f64(x)
    w = _f64(weight)
    b = _f64(bias)
    C = xf.shape[-1]
    N = w.shape[0]
    M = xf.size // C if C else 0
    y = np.zeros(xf.shape[:-1] + (N,), dtype=np.float64)
    rc = _load().oracle_linear(M, C, N, _p(xf), _p(w), _p(b), _p(y))
    _check(rc, "linear")
    return y


def patch_qkv_proj(geom, channels, x, w_qkv, bias=None, k_stale=None, v_stale=None):
    """Q/K/V projection of patch i's hidden states x [B, h, W, C] with
    w_qkv [3C, C] (Q, K, V weights stacked), bias [3C] or None.  Returns
    (q, k, v) as [B, Lq, C] and, for each given stale map [B, H*W, C], a copy
    with patch i's rows replaced by the new k / v (else None)."""
    B, H, W, n, i = geom
    C = channels
    Lq = (H // n) * W
    xf, w, b = _f64(x), _f64(w_qkv), _f64(bias)
    q = np.zeros((B, Lq, C), dtype=np.float64)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    ks = None if k_stale is None else _f64(k_stale).reshape(B, H * W, C).copy()
    vs = None if v_stale is None else _f64(v_stale).reshape(B, H * W, C).copy()
    rc = _load().oracle_patch_qkv_proj(B, H, W, n, i, C, _p(xf), _p(w), _p(b), _p(q), _p(k), _p(v),
                                       _p(ks), _p(vs))
    _check(rc, "patch_qkv_proj")
    return q, k, v, ks, vs
