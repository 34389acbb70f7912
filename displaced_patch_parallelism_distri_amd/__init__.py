"""Python binding of the gfx950 patch-layer library (``libdistri_patch.so``).

One device's share of a DistriFusion patch layer under displaced patch
parallelism: patch self-attention over fresh + stale K/V, the 3x3 conv with a
stale halo, the corrected asynchronous GroupNorm and the stale refresh.  The
functions here only marshal torch tensors (device memory and the current HIP
stream) into the C ABI declared in ``include/distri_patch.h``; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
the library is missing or the call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "DistriError", "load", "abi_version", "geom",
    "distri_patch_self_attn", "distri_patch_conv3x3_halo", "distri_async_groupnorm",
    "distri_refresh_stale", "distri_patch_self_attn_workspace_size",
    "distri_async_groupnorm_workspace_size", "distri_patch_qkv_proj", "distri_patch_out_proj",
    "distri_async_groupnorm_silu", "distri_group_moments", "distri_patch_block",
    "distri_patch_block_sync", "distri_patch_block_workspace_size",
    "distri_patch_block_sync_workspace_size", "BlockWeights", "BlockState",
    "distri_patch_cross_attn", "distri_patch_cross_attn_workspace_size", "naive_geom",
    "distri_async_groupnorm_noalloc", "distri_refresh_stale_maps", "RefreshMap",
    "DISTRI_F32", "DISTRI_BF16", "DISTRI_REFRESH_MAX_MAPS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdistri_patch.so")

DISTRI_F32, DISTRI_BF16 = 0, 1
DISTRI_REFRESH_MAX_MAPS = 8
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_ALIGN",
          5: "ERR_UNSUPPORTED", 6: "ERR_WORKSPACE", 7: "ERR_HIP", 8: "ERR_ALIAS"}
SYMBOLS = ("distri_abi_version", "distri_status_str", "distri_last_error",
           "distri_patch_self_attn_workspace_size", "distri_patch_self_attn",
           "distri_patch_conv3x3_halo", "distri_async_groupnorm_workspace_size",
           "distri_async_groupnorm", "distri_refresh_stale", "distri_patch_qkv_proj",
           "distri_patch_out_proj", "distri_async_groupnorm_silu", "distri_group_moments",
           "distri_patch_block_workspace_size", "distri_patch_block",
           "distri_patch_block_sync_workspace_size", "distri_patch_block_sync",
           "distri_patch_cross_attn_workspace_size", "distri_patch_cross_attn",
           "distri_async_groupnorm_noalloc", "distri_refresh_stale_maps")


class DistriError(RuntimeError):
    def __init__(self, status, func, detail):
        self.status = status
        super().__init__(f"{func}: {STATUS.get(status, status)} ({detail})")


class Geom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("height", ctypes.c_int64), ("width", ctypes.c_int64),
                ("n_patches", ctypes.c_int64), ("patch", ctypes.c_int64)]


class BlockWeights(ctypes.Structure):
    """distri_block_weights: the block's sizes and weight pointers."""
    _fields_ = [("channels", ctypes.c_int64), ("groups", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("eps", ctypes.c_float), ("scale", ctypes.c_float)] + [
        (name, ctypes.c_void_p) for name in ("gn1_gamma", "gn1_beta", "conv_w", "conv_b", "gn2_gamma",
                                             "gn2_beta", "w_qkv", "b_qkv", "w_o", "b_o")]


class RefreshMap(ctypes.Structure):
    """distri_refresh_map: one stale map of distri_refresh_stale_maps."""
    _fields_ = [("rows", ctypes.c_int64), ("row_elems", ctypes.c_int64), ("dtype", ctypes.c_int),
                ("fresh", ctypes.c_void_p), ("stale", ctypes.c_void_p)]


class BlockState(ctypes.Structure):
    """distri_block_state: the stale context maps of one block."""
    _fields_ = [(name, ctypes.c_void_p) for name in ("gn1", "conv_in", "gn2", "k", "v")]


_lib = None


def load():
    """Load libdistri_patch.so (built by ``python -m displaced_patch_parallelism_distri_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m displaced_patch_parallelism_distri_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    G = ctypes.POINTER(Geom)
    lib.distri_abi_version.restype = I
    lib.distri_status_str.restype = ctypes.c_char_p
    lib.distri_status_str.argtypes = [I]
    lib.distri_last_error.restype = ctypes.c_char_p
    lib.distri_patch_self_attn_workspace_size.argtypes = [G, I64, I64, I, ctypes.POINTER(SZ)]
    lib.distri_patch_self_attn.argtypes = [G, I64, I64, ctypes.c_float, I] + [P] * 7 + [SZ, P]
    lib.distri_patch_conv3x3_halo.argtypes = [G, I64, I64, I] + [P] * 5 + [P]
    lib.distri_async_groupnorm_workspace_size.argtypes = [G, I64, I64, I, ctypes.POINTER(SZ)]
    lib.distri_async_groupnorm.argtypes = [G, I64, I64, ctypes.c_float, I] + [P] * 7 + [SZ, P]
    lib.distri_refresh_stale.argtypes = [G, I64, I, P, P, P]
    lib.distri_refresh_stale_maps.argtypes = [G, I, ctypes.POINTER(RefreshMap), P]
    lib.distri_patch_qkv_proj.argtypes = [G, I64, I] + [P] * 9
    lib.distri_patch_out_proj.argtypes = [G, I64, I] + [P] * 5
    lib.distri_async_groupnorm_silu.argtypes = [G, I64, I64, ctypes.c_float, I] + [P] * 7 + [SZ, P]
    lib.distri_async_groupnorm_noalloc.argtypes = [G, I64, I64, ctypes.c_float, I] + [P] * 6 + [P]
    lib.distri_group_moments.argtypes = [G, I64, I64, I, P, P, P, SZ, P]
    BW, BS = ctypes.POINTER(BlockWeights), ctypes.POINTER(BlockState)
    lib.distri_patch_block_workspace_size.argtypes = [G, BW, I, ctypes.POINTER(SZ)]
    lib.distri_patch_block_sync_workspace_size.argtypes = [G, BW, I, ctypes.POINTER(SZ)]
    lib.distri_patch_block.argtypes = [G, BW, I, P, P, BS, BS, P, SZ, P]
    lib.distri_patch_block_sync.argtypes = [G, BW, I, P, P, BS, P, SZ, P]
    lib.distri_patch_cross_attn_workspace_size.argtypes = [G, I64, I64, I64, I, ctypes.POINTER(SZ)]
    lib.distri_patch_cross_attn.argtypes = [G, I64, I64, I64, ctypes.c_float, I] + [P] * 5 + [SZ, P]
    for name in SYMBOLS[3:]:
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load().distri_abi_version())


def geom(batch, height, width, n_patches, patch) -> Geom:
    return Geom(int(batch), int(height), int(width), int(n_patches), int(patch))


def naive_geom(g) -> Geom:
    """The naive-patch baseline's geometry for patch i of ``g``: the patch's
    h rows taken as a whole image (n = 1), so every op sees this patch only:
    attention over its own tokens, zero padding instead of a halo, GroupNorm
    statistics of the patch alone (README mirror, section 概述, figure (b))."""
    g = _as_geom(g)
    return geom(g.batch, g.height // max(g.n_patches, 1), g.width, 1, 0)


def _as_geom(g):
    return g if isinstance(g, Geom) else geom(*g)


def _check(status, func):
    if status != 0:
        detail = load().distri_last_error().decode(errors="replace")
        raise DistriError(status, func, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DISTRI_BF16
    if t.dtype == torch.float32:
        return DISTRI_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _ptr(t, name, dtype=None, numel=None):
    """Device pointer of a dense tensor (or 0 for None)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _record(stream, *tensors):
    """Tensors allocated here (on torch's current stream) but used by a launch
    on another ``stream``: tell the caching allocator, so that it does not
    hand their memory to other work before that stream is done with them."""
    if stream is None:
        return
    ts = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if ts.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None and t.numel() > 0:
            t.record_stream(ts)


def distri_patch_self_attn_workspace_size(g, heads, head_dim, dtype_code) -> int:
    n = ctypes.c_size_t(0)
    _check(load().distri_patch_self_attn_workspace_size(ctypes.byref(_as_geom(g)), heads,
                                                        head_dim, dtype_code, ctypes.byref(n)),
           "distri_patch_self_attn_workspace_size")
    return int(n.value)


def distri_async_groupnorm_workspace_size(g, channels, groups, dtype_code) -> int:
    n = ctypes.c_size_t(0)
    _check(load().distri_async_groupnorm_workspace_size(ctypes.byref(_as_geom(g)), channels,
                                                        groups, dtype_code, ctypes.byref(n)),
           "distri_async_groupnorm_workspace_size")
    return int(n.value)


def _workspace(nbytes, ref, workspace, stream=None):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=ref.device)
        _record(stream, workspace)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace, workspace.numel() * workspace.element_size()


def _new(stream, shape, like, dtype=None):
    """An output tensor allocated here for a launch on ``stream``."""
    t = torch.empty(shape, dtype=like.dtype if dtype is None else dtype, device=like.device)
    _record(stream, t)
    return t


def distri_patch_self_attn(g, heads, q, k_fresh, v_fresh, k_stale, v_stale, out=None,
                           scale=None, head_dim=64, workspace=None, stream=None):
    """Attention of patch i: q/k_fresh/v_fresh [B, Lq, heads, d], k_stale/v_stale
    [B, L, heads, d] -> out [B, Lq, heads, d] (same dtype)."""
    g = _as_geom(g)
    code = _dtype_code(q)
    if out is None:
        out = _new(stream, q.shape, q)
    if scale is None:
        scale = head_dim ** -0.5
    lq = (g.height // max(g.n_patches, 1)) * g.width
    nl = g.batch * lq * heads * head_dim
    nf = g.batch * g.height * g.width * heads * head_dim
    ws_bytes = distri_patch_self_attn_workspace_size(g, heads, head_dim, code)
    ws, ws_len = _workspace(ws_bytes, q, workspace, stream)
    st = load().distri_patch_self_attn(
        ctypes.byref(g), heads, head_dim, float(scale), code,
        _ptr(q, "q", q.dtype, nl), _ptr(k_fresh, "k_fresh", q.dtype, nl),
        _ptr(v_fresh, "v_fresh", q.dtype, nl), _ptr(k_stale, "k_stale", q.dtype, nf),
        _ptr(v_stale, "v_stale", q.dtype, nf), _ptr(out, "out", q.dtype, nl),
        _ptr(ws, "workspace"), ws_len, _stream(stream))
    _check(st, "distri_patch_self_attn")
    return out


def distri_patch_conv3x3_halo(g, x_fresh, x_stale, weight, bias=None, y=None, stream=None):
    """3x3 conv of patch i: x_fresh [B,h,W,Cin], x_stale [B,H,W,Cin], weight
    [Cout,3,3,Cin], bias [Cout] fp32 or None -> y [B,h,W,Cout]."""
    g = _as_geom(g)
    code = _dtype_code(x_fresh)
    cout, cin = weight.shape[0], weight.shape[-1]
    h = g.height // max(g.n_patches, 1)
    if y is None:
        y = _new(stream, (g.batch, h, g.width, cout), x_fresh)
    st = load().distri_patch_conv3x3_halo(
        ctypes.byref(g), cin, cout, code,
        _ptr(x_fresh, "x_fresh", x_fresh.dtype, g.batch * h * g.width * cin),
        _ptr(x_stale, "x_stale", x_fresh.dtype, g.batch * g.height * g.width * cin),
        _ptr(weight, "weight", x_fresh.dtype, cout * 9 * cin),
        _ptr(bias, "bias", torch.float32, cout), _ptr(y, "y", x_fresh.dtype), _stream(stream))
    _check(st, "distri_patch_conv3x3_halo")
    return y


def distri_async_groupnorm(g, groups, x_fresh, stale_moments, gamma=None, beta=None, eps=1e-5,
                           y=None, fresh_moments=None, workspace=None, stream=None):
    """Corrected async GroupNorm of patch i: x_fresh [B,h,W,C], stale_moments
    [B,n,G,2] fp32 -> (y [B,h,W,C], fresh_moments [B,G,2] fp32)."""
    return _groupnorm("distri_async_groupnorm", g, groups, x_fresh, stale_moments, gamma, beta,
                      eps, y, fresh_moments, workspace, stream)


def distri_async_groupnorm_noalloc(g, groups, x_fresh, stale_moments, gamma=None, beta=None,
                                   eps=1e-5, y=None, fresh_moments=None, stream=None):
    """distri_async_groupnorm without a workspace (the library's own 2 MiB
    device scratch; calls that overlap on one GPU race)."""
    g = _as_geom(g)
    code = _dtype_code(x_fresh)
    C = x_fresh.shape[-1]
    if y is None:
        y = _new(stream, x_fresh.shape, x_fresh)
    if fresh_moments is None:
        fresh_moments = _new(stream, (g.batch, groups, 2), x_fresh, torch.float32)
    st = load().distri_async_groupnorm_noalloc(
        ctypes.byref(g), C, groups, float(eps), code, _ptr(x_fresh, "x_fresh", x_fresh.dtype),
        _ptr(stale_moments, "stale_moments", torch.float32, g.batch * g.n_patches * groups * 2),
        _ptr(gamma, "gamma", torch.float32, C), _ptr(beta, "beta", torch.float32, C),
        _ptr(y, "y", x_fresh.dtype, x_fresh.numel()),
        _ptr(fresh_moments, "fresh_moments", torch.float32, g.batch * groups * 2), _stream(stream))
    _check(st, "distri_async_groupnorm_noalloc")
    return y, fresh_moments


def distri_async_groupnorm_silu(g, groups, x_fresh, stale_moments, gamma=None, beta=None,
                                eps=1e-5, y=None, fresh_moments=None, workspace=None, stream=None):
    """distri_async_groupnorm followed by SiLU (same arguments and results)."""
    return _groupnorm("distri_async_groupnorm_silu", g, groups, x_fresh, stale_moments, gamma,
                      beta, eps, y, fresh_moments, workspace, stream)


def distri_group_moments(g, groups, x_fresh, table, workspace=None, stream=None):
    """table[:, i] = raw moments (E[x], E[x^2]) of patch i's x_fresh [B,h,W,C];
    table [B,n,G,2] fp32 is updated in place and returned."""
    g = _as_geom(g)
    code = _dtype_code(x_fresh)
    C = x_fresh.shape[-1]
    ws_bytes = distri_async_groupnorm_workspace_size(g, C, groups, code)
    ws, ws_len = _workspace(ws_bytes, x_fresh, workspace, stream)
    st = load().distri_group_moments(
        ctypes.byref(g), C, groups, code, _ptr(x_fresh, "x_fresh", x_fresh.dtype),
        _ptr(table, "table", torch.float32, g.batch * g.n_patches * groups * 2),
        _ptr(ws, "workspace"), ws_len, _stream(stream))
    _check(st, "distri_group_moments")
    return table


def _groupnorm(func, g, groups, x_fresh, stale_moments, gamma, beta, eps, y, fresh_moments,
               workspace, stream):
    g = _as_geom(g)
    code = _dtype_code(x_fresh)
    C = x_fresh.shape[-1]
    if y is None:
        y = _new(stream, x_fresh.shape, x_fresh)
    if fresh_moments is None:
        fresh_moments = _new(stream, (g.batch, groups, 2), x_fresh, torch.float32)
    ws_bytes = distri_async_groupnorm_workspace_size(g, C, groups, code)
    ws, ws_len = _workspace(ws_bytes, x_fresh, workspace, stream)
    st = getattr(load(), func)(
        ctypes.byref(g), C, groups, float(eps), code, _ptr(x_fresh, "x_fresh", x_fresh.dtype),
        _ptr(stale_moments, "stale_moments", torch.float32, g.batch * g.n_patches * groups * 2),
        _ptr(gamma, "gamma", torch.float32, C), _ptr(beta, "beta", torch.float32, C),
        _ptr(y, "y", x_fresh.dtype, x_fresh.numel()),
        _ptr(fresh_moments, "fresh_moments", torch.float32, g.batch * groups * 2),
        _ptr(ws, "workspace"), ws_len, _stream(stream))
    _check(st, func)
    return y, fresh_moments


def distri_refresh_stale(g, row_elems, fresh, stale, stream=None):
    """stale[b, i*h + r, :] = fresh[b, r, :] in place; returns stale."""
    g = _as_geom(g)
    code = _dtype_code(fresh)
    h = g.height // max(g.n_patches, 1)
    st = load().distri_refresh_stale(
        ctypes.byref(g), row_elems, code,
        _ptr(fresh, "fresh", fresh.dtype, g.batch * h * row_elems),
        _ptr(stale, "stale", fresh.dtype, g.batch * g.height * row_elems), _stream(stream))
    _check(st, "distri_refresh_stale")
    return stale


def distri_refresh_stale_maps(g, maps, stream=None):
    """All of a layer's stale maps in one launch.  ``maps`` is a sequence of
    (rows, row_elems, fresh, stale): per image, fresh [B, rows, row_elems]
    goes to rows [i*rows, (i+1)*rows) of stale [B, n*rows, row_elems]
    (rows = H/n for feature and K/V maps, 1 for a GroupNorm moment table).
    Returns the stale tensors."""
    g = _as_geom(g)
    arr = (RefreshMap * max(len(maps), 1))()
    for k, (rows, row_elems, fresh, stale) in enumerate(maps):
        code = _dtype_code(fresh)
        arr[k] = RefreshMap(rows, row_elems, code,
                            _ptr(fresh, "fresh", fresh.dtype, g.batch * rows * row_elems),
                            _ptr(stale, "stale", fresh.dtype, g.batch * g.n_patches * rows * row_elems))
    st = load().distri_refresh_stale_maps(ctypes.byref(g), len(maps), arr, _stream(stream))
    _check(st, "distri_refresh_stale_maps")
    return [m[3] for m in maps]


def distri_patch_qkv_proj(g, x, w_qkv, bias=None, q=None, k_fresh=None, v_fresh=None, k_stale=None,
                          v_stale=None, stream=None):
    """Q/K/V projection of patch i: x [B, h, W, C] (or [B, Lq, C]), w_qkv
    [3C, C], bias [3C] fp32 or None -> (q, k_fresh, v_fresh), each [B, Lq, C];
    k_stale / v_stale [B, H*W, C] (optional) get patch i's rows of k / v."""
    g = _as_geom(g)
    code = _dtype_code(x)
    C = x.shape[-1]
    lq = (g.height // max(g.n_patches, 1)) * g.width
    shape = (g.batch, lq, C)
    q = _new(stream, shape, x) if q is None else q
    k_fresh = _new(stream, shape, x) if k_fresh is None else k_fresh
    v_fresh = _new(stream, shape, x) if v_fresh is None else v_fresh
    n_tok = g.batch * lq * C
    n_full = g.batch * g.height * g.width * C
    st = load().distri_patch_qkv_proj(
        ctypes.byref(g), C, code, _ptr(x, "x", x.dtype, n_tok), _ptr(w_qkv, "w_qkv", x.dtype, 3 * C * C),
        _ptr(bias, "bias", torch.float32, 3 * C), _ptr(q, "q", x.dtype, n_tok),
        _ptr(k_fresh, "k_fresh", x.dtype, n_tok), _ptr(v_fresh, "v_fresh", x.dtype, n_tok),
        _ptr(k_stale, "k_stale", x.dtype, n_full), _ptr(v_stale, "v_stale", x.dtype, n_full),
        _stream(stream))
    _check(st, "distri_patch_qkv_proj")
    return q, k_fresh, v_fresh


def distri_patch_out_proj(g, o, w_o, bias=None, y=None, stream=None):
    """Output projection of patch i: o [B, Lq, C] (or [B, Lq, heads, d]),
    w_o [C, C], bias [C] fp32 or None -> y [B, Lq, C]."""
    g = _as_geom(g)
    code = _dtype_code(o)
    C = w_o.shape[0]
    lq = (g.height // max(g.n_patches, 1)) * g.width
    if y is None:
        y = _new(stream, (g.batch, lq, C), o)
    n_tok = g.batch * lq * C
    st = load().distri_patch_out_proj(
        ctypes.byref(g), C, code, _ptr(o, "o", o.dtype, n_tok), _ptr(w_o, "w_o", o.dtype, C * C),
        _ptr(bias, "bias", torch.float32, C), _ptr(y, "y", o.dtype, n_tok), _stream(stream))
    _check(st, "distri_patch_out_proj")
    return y


# ------------------------------------------------------------------ the block
_WEIGHT_KEYS = ("gn1_gamma", "gn1_beta", "conv_w", "conv_b", "gn2_gamma", "gn2_beta", "w_qkv",
                "b_qkv", "w_o", "b_o")
_STATE_KEYS = ("gn1", "conv_in", "gn2", "k", "v")


def _block_weights(weights, channels, groups, heads, eps, scale, dtype):
    """BlockWeights from a dict of device tensors (fp32 vectors; conv_w
    [C,3,3,C], w_qkv [3C,C], w_o [C,C] in the activation dtype)."""
    C = channels
    sizes = {"gn1_gamma": C, "gn1_beta": C, "conv_b": C, "gn2_gamma": C, "gn2_beta": C,
             "b_qkv": 3 * C, "b_o": C, "conv_w": 9 * C * C, "w_qkv": 3 * C * C, "w_o": C * C}
    bw = BlockWeights(int(channels), int(groups), int(heads), float(eps),
                      float(scale if scale is not None else 64 ** -0.5))
    for k in _WEIGHT_KEYS:
        t = weights.get(k)
        dt = dtype if k in ("conv_w", "w_qkv", "w_o") else torch.float32
        setattr(bw, k, _ptr(t, k, dt, sizes[k]))
    return bw


def _block_state(state, g, channels, groups, dtype):
    B, H, W, n = g.batch, g.height, g.width, g.n_patches
    sizes = {"gn1": B * n * groups * 2, "gn2": B * n * groups * 2,
             "conv_in": B * H * W * channels, "k": B * H * W * channels, "v": B * H * W * channels}
    bs = BlockState()
    for k in _STATE_KEYS:
        dt = torch.float32 if k in ("gn1", "gn2") else dtype
        setattr(bs, k, _ptr(state[k], "state " + k, dt, sizes[k]))
    return bs


def distri_patch_block_workspace_size(g, channels, groups, heads, dtype_code, sync=False) -> int:
    bw = BlockWeights(int(channels), int(groups), int(heads), 1e-5, 0.125)
    n = ctypes.c_size_t(0)
    func = "distri_patch_block_sync_workspace_size" if sync else "distri_patch_block_workspace_size"
    _check(getattr(load(), func)(ctypes.byref(_as_geom(g)), ctypes.byref(bw), dtype_code,
                                 ctypes.byref(n)), func)
    return int(n.value)


def distri_patch_block_sync_workspace_size(g, channels, groups, heads, dtype_code) -> int:
    return distri_patch_block_workspace_size(g, channels, groups, heads, dtype_code, sync=True)


def distri_patch_block(g, weights, x, state_in, state_out=None, y=None, groups=32, heads=None,
                       eps=1e-5, scale=None, workspace=None, stream=None):
    """One asynchronous step of the block for patch i.  x [B,h,W,C] -> y
    [B,Lq,C]; state_in / state_out: dicts with gn1, gn2 [B,n,G,2] fp32,
    conv_in [B,H,W,C], k, v [B,H*W,C] (state_out defaults to state_in:
    updated in place)."""
    g = _as_geom(g)
    code = _dtype_code(x)
    C = x.shape[-1]
    heads = C // 64 if heads is None else heads
    if y is None:
        y = _new(stream, (g.batch, (g.height // max(g.n_patches, 1)) * g.width, C), x)
    bw = _block_weights(weights, C, groups, heads, eps, scale, x.dtype)
    sin = _block_state(state_in, g, C, groups, x.dtype)
    sout = sin if state_out is None else _block_state(state_out, g, C, groups, x.dtype)
    ws_bytes = distri_patch_block_workspace_size(g, C, groups, heads, code)
    ws, ws_len = _workspace(ws_bytes, x, workspace, stream)
    st = load().distri_patch_block(
        ctypes.byref(g), ctypes.byref(bw), code, _ptr(x, "x", x.dtype, y.numel()),
        _ptr(y, "y", x.dtype, y.numel()), ctypes.byref(sin), ctypes.byref(sout),
        _ptr(ws, "workspace"), ws_len, _stream(stream))
    _check(st, "distri_patch_block")
    return y


def distri_patch_block_sync(g, weights, x, state, y=None, groups=32, heads=None, eps=1e-5,
                            scale=None, workspace=None, stream=None):
    """The synchronous (warm-up) step for all n patches on one device.
    x [n, B, h, W, C] (patch-major) -> y [n, B, Lq, C]; fills ``state``."""
    g = _as_geom(g)
    code = _dtype_code(x)
    C = x.shape[-1]
    heads = C // 64 if heads is None else heads
    n = g.n_patches
    lq = (g.height // max(n, 1)) * g.width
    if y is None:
        y = _new(stream, (n, g.batch, lq, C), x)
    bw = _block_weights(weights, C, groups, heads, eps, scale, x.dtype)
    bs = _block_state(state, g, C, groups, x.dtype)
    ws_bytes = distri_patch_block_sync_workspace_size(g, C, groups, heads, code)
    ws, ws_len = _workspace(ws_bytes, x, workspace, stream)
    st = load().distri_patch_block_sync(
        ctypes.byref(g), ctypes.byref(bw), code, _ptr(x, "x", x.dtype, y.numel()),
        _ptr(y, "y", x.dtype, y.numel()), ctypes.byref(bs), _ptr(ws, "workspace"), ws_len,
        _stream(stream))
    _check(st, "distri_patch_block_sync")
    return y


def distri_patch_cross_attn_workspace_size(g, heads, ctx_len, dtype_code, head_dim=64) -> int:
    n = ctypes.c_size_t(0)
    _check(load().distri_patch_cross_attn_workspace_size(ctypes.byref(_as_geom(g)), heads, head_dim,
                                                         ctx_len, dtype_code, ctypes.byref(n)),
           "distri_patch_cross_attn_workspace_size")
    return int(n.value)


def distri_patch_cross_attn(g, heads, q, k_ctx, v_ctx, out=None, scale=None, head_dim=64,
                            workspace=None, stream=None):
    """Cross-attention of patch i: q [B, Lq, heads, d] over a shared context
    k_ctx, v_ctx [B, ctx_len, heads, d] -> out [B, Lq, heads, d]."""
    g = _as_geom(g)
    code = _dtype_code(q)
    ctx_len = k_ctx.shape[1]
    if out is None:
        out = _new(stream, q.shape, q)
    if scale is None:
        scale = head_dim ** -0.5
    lq = (g.height // max(g.n_patches, 1)) * g.width
    nl = g.batch * lq * heads * head_dim
    nc = g.batch * ctx_len * heads * head_dim
    ws_bytes = distri_patch_cross_attn_workspace_size(g, heads, ctx_len, code, head_dim)
    ws, ws_len = _workspace(ws_bytes, q, workspace, stream)
    st = load().distri_patch_cross_attn(
        ctypes.byref(g), heads, head_dim, ctx_len, float(scale), code, _ptr(q, "q", q.dtype, nl),
        _ptr(k_ctx, "k_ctx", q.dtype, nc), _ptr(v_ctx, "v_ctx", q.dtype, nc),
        _ptr(out, "out", q.dtype, nl), _ptr(ws, "workspace"), ws_len, _stream(stream))
    _check(st, "distri_patch_cross_attn")
    return out
