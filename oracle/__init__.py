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
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_patch_self_attn.argtypes = [_I] * 7 + [ctypes.c_double] + [_D] * 5 + [_I, _I, _D]
        lib.oracle_patch_conv3x3_halo.argtypes = [_I] * 7 + [_D] * 4 + [_I, _I, _D]
        lib.oracle_group_moments.argtypes = [_I] * 5 + [_D, _D]
        lib.oracle_async_groupnorm.argtypes = [_I] * 7 + [ctypes.c_double] + [_D] * 6
        lib.oracle_refresh_stale.argtypes = [_I] * 5 + [_D, _D]
        lib.oracle_linear.argtypes = [_I] * 3 + [_D] * 4
        lib.oracle_patch_qkv_proj.argtypes = [_I] * 6 + [_D] * 8
        lib.oracle_silu.argtypes = [_I, _D, _D]
        lib.oracle_cross_attn.argtypes = [_I] * 5 + [ctypes.c_double] + [_D] * 4
        for f in ("oracle_patch_self_attn", "oracle_patch_conv3x3_halo", "oracle_group_moments",
                  "oracle_async_groupnorm", "oracle_refresh_stale", "oracle_linear",
                  "oracle_patch_qkv_proj", "oracle_silu", "oracle_cross_attn"):
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


def set_num_threads(n: int) -> None:
    """OpenMP threads of the calls that follow (for timing only)."""
    _load().oracle_set_num_threads(int(n))


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


def cross_attn(scale, q, k_ctx, v_ctx):
    """Patch queries q [B, Lq, heads, d] over a shared context k_ctx, v_ctx
    [B, Lk, heads, d] -> [B, Lq, heads, d] float64."""
    qf, kf, vf = _f64(q), _f64(k_ctx), _f64(v_ctx)
    B, Lq, heads, d = qf.shape
    Lk = kf.shape[1]
    out = np.zeros((B, Lq, heads, d), dtype=np.float64)
    _check(_load().oracle_cross_attn(B, Lq, Lk, heads, d, float(scale), _p(qf), _p(kf), _p(vf), _p(out)),
           "cross_attn")
    return out


def round_to(a, dtype):
    """Every value rounded to the nearest value of ``dtype``, ties to even,
    returned as float64: "bf16" keeps 8 significant bits (the upper half of
    an IEEE binary32), "f32" is binary32.  This is storage rounding, applied
    where a chain of ops hands a tensor of that dtype to the next op (bf16
    results of these ops stay far inside binary32's exponent range, so bf16
    subnormals and overflow are not handled)."""
    a = _f64(a)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    m, e = np.frexp(a)                       # a = m 2^e with 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # np.rint: ties to even


def silu(z):
    """Elementwise z / (1 + exp(-z)), float64, same shape."""
    zf = _f64(z)
    y = np.zeros_like(zf)
    _check(_load().oracle_silu(zf.size, _p(zf), _p(y)), "silu")
    return y


# ---------------------------------------------------------------- patch block
# The wrapped layers chained at patch granularity for one denoising step
# ("DistriFusion源码探秘", section "Patch Parallelism的实现原理": conv,
# self-attention and GroupNorm are the wrapped layer types):
#   g1 = SiLU(GN1(x)); h = conv3x3(g1) + b; n2 = GN2(h);
#   q, k, v = n2 Wqkv^T + b; o = softmax(scale q K^T) V; y = o Wo^T + b.
# ``wts`` is a dict: channels, groups, heads, eps, scale, gn1_gamma, gn1_beta,
# conv_w [C,3,3,C], conv_b, gn2_gamma, gn2_beta, w_qkv [3C,C], b_qkv, w_o
# [C,C], b_o.  A state is a dict of the previous step's context: gn1, gn2
# [B, n, G, 2] moment tables, conv_in [B, H, W, C] (g1 of every patch), k, v
# [B, H*W, C].  These functions only sequence the C routines above.
#
# ``act_dtype``: None chains the ops in float64 throughout.  "bf16" or "f32"
# gives every op its inputs as tensors of that dtype, as a chain of the
# library's ops holds them: each op's result is rounded (round_to) before the
# next op reads it, and the results returned (y and the new state rows) are
# each op's own result before that rounding.

def _rounder(act_dtype):
    return (lambda a: a) if act_dtype is None else (lambda a: round_to(a, act_dtype))


def patch_block(geom, wts, x, state, act_dtype=None):
    """One asynchronous step for patch i: x [B, h, W, C] -> (y [B, Lq, C],
    new state).  Stale reads come from ``state``; the new state is a copy
    with patch i's rows / slots replaced by this step's fresh values (README
    mirror, section 概述, figure (c): the next step reuses them)."""
    B, H, W, n, i = geom
    C, G, nh = wts["channels"], wts["groups"], wts["heads"]
    h, Lq, L, d = H // n, (H // n) * W, H * W, C // nh
    r = _rounder(act_dtype)
    z1, fm1 = async_groupnorm(geom, C, G, wts["eps"], x, state["gn1"], wts["gn1_gamma"],
                              wts["gn1_beta"])
    g1 = silu(z1)
    hh = patch_conv3x3_halo(geom, C, C, r(g1), state["conv_in"], wts["conv_w"], wts["conv_b"])
    n2, fm2 = async_groupnorm(geom, C, G, wts["eps"], r(hh), state["gn2"], wts["gn2_gamma"],
                              wts["gn2_beta"])
    q, k, v, ks, vs = patch_qkv_proj(geom, C, r(n2), wts["w_qkv"], wts["b_qkv"], state["k"], state["v"])
    o = patch_self_attn(geom, nh, d, wts["scale"], r(q).reshape(B, Lq, nh, d),
                        r(k).reshape(B, Lq, nh, d), r(v).reshape(B, Lq, nh, d),
                        _f64(state["k"]).reshape(B, L, nh, d), _f64(state["v"]).reshape(B, L, nh, d))
    y = linear(r(o).reshape(B, Lq, C), wts["w_o"], wts["b_o"])
    tgeom = (B, n, 1, n, i)
    new = {
        "gn1": refresh_stale(tgeom, 2 * G, fm1.reshape(B, 1, 2 * G),
                             _f64(state["gn1"]).reshape(B, n, 2 * G)).reshape(B, n, G, 2),
        "conv_in": refresh_stale(geom, W * C, g1.reshape(B, h, W * C),
                                 _f64(state["conv_in"]).reshape(B, H, W * C)).reshape(B, H, W, C),
        "gn2": refresh_stale(tgeom, 2 * G, fm2.reshape(B, 1, 2 * G),
                             _f64(state["gn2"]).reshape(B, n, 2 * G)).reshape(B, n, G, 2),
        "k": ks,
        "v": vs,
    }
    return y, new


def patch_block_sync(geom, wts, x_full, act_dtype=None):
    """The synchronous (warm-up) step for all n patches: each stage runs for
    every patch, and its fresh values are shared, before any patch reads
    them in the next stage (the first denoising steps exchange activations
    synchronously: README mirror, section 概述, figure (c)).
    x_full [B, H, W, C] -> (y [B, H*W, C], state of this step)."""
    B, H, W, n, _ = geom
    C, G, nh = wts["channels"], wts["groups"], wts["heads"]
    h, Lq, L, d = H // n, (H // n) * W, H * W, C // nh
    r = _rounder(act_dtype)
    xf = _f64(x_full)
    geoms = [(B, H, W, n, j) for j in range(n)]
    rows = [slice(j * h, (j + 1) * h) for j in range(n)]
    toks = [slice(j * Lq, (j + 1) * Lq) for j in range(n)]
    eps = wts["eps"]

    gn1 = np.zeros((B, n, G, 2))
    for j in range(n):
        gn1[:, j] = group_moments(xf[:, rows[j]], G)
    g1 = [silu(async_groupnorm(geoms[j], C, G, eps, xf[:, rows[j]], gn1, wts["gn1_gamma"],
                               wts["gn1_beta"])[0]) for j in range(n)]
    conv_in = np.zeros((B, H * W * C))
    for j in range(n):
        conv_in = refresh_stale(geoms[j], W * C, g1[j].reshape(B, h, W * C),
                                conv_in.reshape(B, H, W * C))
    conv_in = conv_in.reshape(B, H, W, C)
    hh = [r(patch_conv3x3_halo(geoms[j], C, C, r(g1[j]), r(conv_in), wts["conv_w"], wts["conv_b"]))
          for j in range(n)]
    gn2 = np.zeros((B, n, G, 2))
    for j in range(n):
        gn2[:, j] = group_moments(hh[j], G)
    n2 = [r(async_groupnorm(geoms[j], C, G, eps, hh[j], gn2, wts["gn2_gamma"], wts["gn2_beta"])[0])
          for j in range(n)]
    kmap = np.zeros((B, L, C))
    vmap = np.zeros((B, L, C))
    qkv = []
    for j in range(n):
        q, k, v, kmap, vmap = patch_qkv_proj(geoms[j], C, n2[j], wts["w_qkv"], wts["b_qkv"], kmap, vmap)
        qkv.append((r(q), r(k), r(v)))
    y = np.zeros((B, L, C))
    for j in range(n):
        q, k, v = (t.reshape(B, Lq, nh, d) for t in qkv[j])
        o = patch_self_attn(geoms[j], nh, d, wts["scale"], q, k, v, r(kmap).reshape(B, L, nh, d),
                            r(vmap).reshape(B, L, nh, d))
        y[:, toks[j]] = linear(r(o).reshape(B, Lq, C), wts["w_o"], wts["b_o"])
    state = {"gn1": gn1, "conv_in": conv_in, "gn2": gn2, "k": kmap, "v": vmap}
    return y, state
