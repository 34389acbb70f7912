"""C-ABI boundary checks that need no GPU.

The library must load, export every entry point the header declares, and
reject every invalid argument with its status code before any HIP call - so
these calls are safe without a device: the fake pointers are never touched.
"""
import ctypes
import os
import re

import pytest

import displaced_patch_parallelism_distri_amd as dp

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "distri_patch.h")
OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, HIP, ALIAS = range(9)
BF16, F32 = dp.DISTRI_BF16, dp.DISTRI_F32
A = 0x7f0000000000  # a fake, 16-byte aligned "device" address, never dereferenced
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    return dp.load()


def G(*v):
    return ctypes.byref(dp.geom(*v))


def test_exports_every_declared_symbol(lib):
    with open(HEADER) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:int|const char \*|size_t)\s*(distri_\w+)\s*\(", text, re.M))
    assert declared == set(dp.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert dp.abi_version() == 1
    assert lib.distri_status_str(OK) == b"ok"
    assert lib.distri_status_str(ALIAS) == b"output overlaps an input"
    assert lib.distri_status_str(99) == b"unknown status"


def attn(lib, geom, heads=10, hd=64, scale=0.125, dtype=BF16, ptrs=None, ws=None, wsb=0):
    p = ptrs or [A + k * 64 * MB for k in range(6)]
    return lib.distri_patch_self_attn(G(*geom), heads, hd, scale, dtype, *p, ws, wsb, None)


def test_attention_rejects_bad_arguments(lib):
    g = (2, 64, 64, 8, 3)
    assert lib.distri_patch_self_attn(None, 10, 64, 0.125, BF16, *([A] * 6), None, 0, None) == NULL
    assert attn(lib, (2, 65, 64, 8, 0)) == SHAPE          # H % n != 0
    assert attn(lib, (2, 64, 64, 8, 8)) == SHAPE          # i >= n
    assert attn(lib, (2, 64, 64, 0, 0)) == SHAPE          # n < 1
    assert attn(lib, (-1, 64, 64, 8, 0)) == SHAPE
    assert attn(lib, g, hd=128) == UNSUP                  # head_dim != 64
    assert attn(lib, g, heads=0) == SHAPE
    assert attn(lib, g, dtype=7) == DTYPE
    assert attn(lib, g, scale=0.0) == SHAPE
    assert attn(lib, g, scale=float("inf")) == SHAPE
    p = [A + k * 64 * MB for k in range(6)]
    p[2] = None
    assert attn(lib, g, ptrs=p) == NULL
    p = [A + k * 64 * MB for k in range(6)]
    p[4] += 8
    assert attn(lib, g, ptrs=p) == ALIGN
    p = [A + k * 64 * MB for k in range(6)]
    p[5] = p[3] + 1024                                   # out inside k_stale
    assert attn(lib, g, ptrs=p) == ALIAS


def test_attention_empty_output_is_ok_without_pointers(lib):
    assert attn(lib, (0, 64, 64, 8, 0), ptrs=[None] * 6) == OK
    assert attn(lib, (2, 0, 64, 8, 0), ptrs=[None] * 6) == OK


def test_attention_workspace_size_needs_no_device(lib):
    """The key-split plan is made for a fixed 256-CU machine, so the size is a
    function of the sizes alone (and nonzero where tasks are split)."""
    g = (2, 240, 240, 8, 4)
    n = dp.distri_patch_self_attn_workspace_size(g, 10, 64, BF16)
    # 44 leftover tasks x 17 key chunks x 512 queries x (64 + 2) fp32
    assert n == 44 * 17 * 512 * 66 * 4
    assert dp.distri_patch_self_attn_workspace_size(g, 10, 64, F32) == 0
    assert n == dp.distri_patch_self_attn_workspace_size(g, 10, 64, BF16)


def test_attention_rejects_small_or_overlapping_workspace(lib):
    g = (2, 240, 240, 8, 4)
    need = dp.distri_patch_self_attn_workspace_size(g, 10, 64, BF16)
    full = 2 * 240 * 240 * 640 * 2
    p = [A + k * 4 * full for k in range(6)]
    ws = A + 24 * full
    assert attn(lib, g, ptrs=p, ws=None, wsb=0) == WS
    assert attn(lib, g, ptrs=p, ws=ws, wsb=need - 16) == WS
    assert attn(lib, g, ptrs=p, ws=ws + 8, wsb=need) == ALIGN
    for k in range(6):                       # q, k_fresh, v_fresh, k_stale, v_stale, out
        assert attn(lib, g, ptrs=p, ws=p[k] + 256, wsb=need) == ALIAS, k


def test_cross_attention_rejects_overlapping_workspace(lib):
    g = (2, 64, 64, 8, 3)
    ctx = 300                                # past the on-chip context: a workspace is needed
    need = dp.distri_patch_cross_attn_workspace_size(g, 10, ctx, BF16)
    assert need > 0
    p = [A + k * 64 * MB for k in range(4)]  # q, k_ctx, v_ctx, out
    for k in range(4):
        st = lib.distri_patch_cross_attn(G(*g), 10, 64, ctx, 0.125, BF16, *p, p[k] + 256, need, None)
        assert st == ALIAS, k
    st = lib.distri_patch_cross_attn(G(*g), 10, 64, ctx, 0.125, BF16, *p, A + 8 * 64 * MB, need - 16, None)
    assert st == WS


def conv(lib, geom, cin=640, cout=640, dtype=BF16, ptrs=None, bias=None):
    p = ptrs or [A + k * 256 * MB for k in range(4)]
    return lib.distri_patch_conv3x3_halo(G(*geom), cin, cout, dtype, p[0], p[1], p[2], bias, p[3], None)


def test_conv_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    assert conv(lib, (2, 241, 240, 8, 4)) == SHAPE
    assert conv(lib, (2, 240, 240, 8, 9)) == SHAPE
    assert conv(lib, g, cin=48) == UNSUP                  # bf16 needs c_in % 64
    assert conv(lib, g, cin=96) == UNSUP
    assert conv(lib, g, cin=0) == SHAPE
    assert conv(lib, g, dtype=2) == DTYPE
    assert conv(lib, g, ptrs=[A, None, A + 512 * MB, A + 768 * MB]) == NULL   # stale needed (n > 1)
    assert conv(lib, g, ptrs=[A, A + 256 * MB, A + 512 * MB, A + 8]) == ALIGN
    assert conv(lib, g, ptrs=[A, A + 256 * MB, A + 512 * MB, A + 16]) == ALIAS
    assert conv(lib, g, bias=A + 4) == ALIGN
    assert conv(lib, (0, 240, 240, 8, 4), ptrs=[None] * 4) == OK


def test_groupnorm_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    n = ctypes.c_size_t(0)
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 640, 32, BF16, ctypes.byref(n)) == OK
    assert n.value > 0
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 640, 33, BF16, ctypes.byref(n)) == SHAPE
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 644, 4, BF16, ctypes.byref(n)) == UNSUP
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 2048, 512, BF16, ctypes.byref(n)) == UNSUP
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 2048, 256, BF16, ctypes.byref(n)) == OK
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 640, 32, BF16, None) == NULL
    x, tab, gam, bet, y, fm, ws = (A + k * 64 * MB for k in range(7))

    def call(geom=g, C=640, G_=32, eps=1e-5, dt=BF16, x=x, tab=tab, y=y, fm=fm, ws=ws, wsb=n.value):
        return lib.distri_async_groupnorm(G(*geom), C, G_, eps, dt, x, tab, gam, bet, y, fm, ws, wsb, None)

    lib.distri_async_groupnorm_workspace_size(G(*g), 640, 32, BF16, ctypes.byref(n))
    assert call(eps=-1.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(wsb=n.value - 1) == WS
    assert call(ws=None) == WS
    assert call(tab=None) == NULL
    assert call(fm=A + 64 * MB * 5 + 4) == ALIGN
    assert call(y=x + 1024) == ALIAS
    assert call(ws=y + 16) == ALIAS
    assert call(geom=(2, 240, 240, 7, 0)) == SHAPE
    assert call(geom=(0, 240, 240, 8, 0), x=None, tab=None, y=None, fm=None, ws=None) == OK


def test_refresh_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    f, s = A, A + 512 * MB
    assert lib.distri_refresh_stale(G(*g), -1, BF16, f, s, None) == SHAPE
    assert lib.distri_refresh_stale(G(*g), 100, 5, f, s, None) == DTYPE
    assert lib.distri_refresh_stale(G(*g), 100, BF16, None, s, None) == NULL
    assert lib.distri_refresh_stale(G(*g), 100, BF16, f + 1, s, None) == ALIGN
    assert lib.distri_refresh_stale(G(*g), 100, F32, f + 2, s, None) == ALIGN
    assert lib.distri_refresh_stale(G(*g), 100, BF16, f, f + 2, None) == ALIAS
    assert lib.distri_refresh_stale(G(*(2, 240, 240, 8, 8)), 100, BF16, f, s, None) == SHAPE
    assert lib.distri_refresh_stale(G(*g), 0, BF16, None, None, None) == OK


def maps_of(*entries):
    arr = (dp.RefreshMap * max(len(entries), 1))()
    for k, e in enumerate(entries):
        arr[k] = dp.RefreshMap(*e)
    return arr


def test_refresh_maps_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    h, W, C = 30, 240, 640
    kv = (h, W * C, BF16, A, A + 512 * MB)            # a [2, 240, 240, 640] map, patch rows h
    tab = (1, 64, F32, A + 1024 * MB, A + 1025 * MB)  # a [2, 8, 32, 2] moment table
    call = lambda *e, count=None: lib.distri_refresh_stale_maps(
        G(*g), len(e) if count is None else count, maps_of(*e), None)
    assert lib.distri_refresh_stale_maps(G(*g), 0, None, None) == OK
    assert lib.distri_refresh_stale_maps(G(*g), 2, None, None) == NULL
    assert lib.distri_refresh_stale_maps(None, 1, maps_of(kv), None) == NULL
    assert call(kv, count=-1) == SHAPE
    assert call(*([kv] * 9)) == UNSUP                 # more than DISTRI_REFRESH_MAX_MAPS
    assert call((h, W * C, 7, A, A + 512 * MB)) == DTYPE
    assert call((-1, W * C, BF16, A, A + 512 * MB)) == SHAPE
    assert call((h, W * C, BF16, None, A + 512 * MB)) == NULL
    assert call((h, W * C, BF16, A + 1, A + 512 * MB)) == ALIGN
    assert call((1, 64, F32, A + 2, A + 512 * MB)) == ALIGN
    assert call(kv, (h, W * C, BF16, A + 256 * MB, A + 512 * MB + 64)) == ALIAS   # stale maps overlap
    assert call(kv, (h, W * C, BF16, A + 512 * MB + 64, A + 2048 * MB)) == ALIAS  # a fresh in a stale
    assert lib.distri_refresh_stale_maps(G(2, 240, 240, 8, 8), 1, maps_of(kv), None) == SHAPE
    assert call((0, W * C, BF16, None, None), (h, 0, BF16, None, None)) == OK  # empty maps: nothing to do
    assert lib.distri_refresh_stale_maps(G(0, 240, 240, 8, 4), 2, maps_of(kv, tab), None) == OK


def test_last_error_names_the_argument(lib):
    attn(lib, (2, 64, 64, 8, 0), hd=32)
    assert b"head_dim" in lib.distri_last_error()


def test_python_binding_raises_on_cpu_tensors():
    import torch

    x = torch.zeros(2, 8, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        dp.distri_refresh_stale((2, 32, 8, 4, 0), 8 * 64, x, torch.zeros(2, 32, 8, 64, dtype=torch.bfloat16))


def qkv(lib, geom, C=640, dtype=BF16, ptrs=None, bias=None):
    p = ptrs or [A + k * 512 * MB for k in range(7)]
    x, w, q, k, v, ks, vs = p
    return lib.distri_patch_qkv_proj(G(*geom), C, dtype, x, w, bias, q, k, v, ks, vs, None)


def test_qkv_proj_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    assert qkv(lib, (2, 240, 240, 8, 8)) == SHAPE
    assert qkv(lib, g, C=0) == SHAPE
    assert qkv(lib, g, C=96) == UNSUP                    # bf16 needs C % 64 == 0
    assert qkv(lib, g, C=65600) == UNSUP
    assert qkv(lib, g, dtype=3) == DTYPE
    assert qkv(lib, (70000, 240, 240, 8, 4)) == UNSUP    # B * Lq >= 2^31
    assert qkv(lib, (1, 1 << 22, 4096, 1024, 0), C=65536) == UNSUP  # grid too large
    p = [A + k * 512 * MB for k in range(7)]
    p[1] = None
    assert qkv(lib, g, ptrs=p) == NULL
    p = [A + k * 512 * MB for k in range(7)]
    p[4] += 8
    assert qkv(lib, g, ptrs=p) == ALIGN
    assert qkv(lib, g, bias=A + 7 * 512 * MB + 4) == ALIGN
    p = [A + k * 512 * MB for k in range(7)]
    p[3] = p[0] + 1024                                   # k inside x
    assert qkv(lib, g, ptrs=p) == ALIAS
    p = [A + k * 512 * MB for k in range(7)]
    p[6] = p[5] + 1024                                   # the two stale maps overlap
    assert qkv(lib, g, ptrs=p) == ALIAS
    p = [A + k * 512 * MB for k in range(7)]
    assert qkv(lib, g, bias=p[2] + 64) == ALIAS          # q written over the bias
    assert qkv(lib, (0, 240, 240, 8, 4), ptrs=[None] * 7) == OK


def test_out_proj_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    o, w, y = A, A + 512 * MB, A + 1024 * MB

    def call(geom=g, C=640, dtype=BF16, o=o, w=w, bias=None, y=y):
        return lib.distri_patch_out_proj(G(*geom), C, dtype, o, w, bias, y, None)

    assert call(C=-1) == SHAPE
    assert call(C=32) == UNSUP
    assert call(dtype=9) == DTYPE
    assert call(o=None) == NULL
    assert call(y=y + 2) == ALIGN
    assert call(y=o + 4096) == ALIAS
    assert call(bias=y + 256) == ALIAS
    assert call(geom=(2, 241, 240, 8, 4)) == SHAPE
    assert call(geom=(2, 240, 0, 8, 4), o=None, w=None, y=None) == OK


def test_groupnorm_variants_reject_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    n = ctypes.c_size_t(0)
    assert lib.distri_async_groupnorm_workspace_size(G(*g), 640, 32, BF16, ctypes.byref(n)) == OK
    x, tab, y, fm, ws = (A + k * 64 * MB for k in range(5))
    call = lambda **kw: lib.distri_async_groupnorm_silu(
        G(*kw.get("geom", g)), kw.get("C", 640), kw.get("G", 32), kw.get("eps", 1e-5), BF16,
        kw.get("x", x), kw.get("tab", tab), None, None, kw.get("y", y), kw.get("fm", fm),
        kw.get("ws", ws), kw.get("wsb", n.value), None)
    assert call(C=630) == SHAPE
    assert call(G=512, C=1024) == UNSUP
    assert call(tab=None) == NULL
    assert call(wsb=n.value - 1) == WS
    assert call(y=x + 64) == ALIAS
    mom = lambda **kw: lib.distri_group_moments(
        G(*kw.get("geom", g)), 640, 32, BF16, kw.get("x", x), kw.get("tab", tab), kw.get("ws", ws),
        kw.get("wsb", n.value), None)
    assert mom(tab=None) == NULL
    assert mom(tab=tab + 4) == ALIGN
    assert mom(wsb=0) == WS
    assert mom(tab=x + 1024) == ALIAS
    assert mom(ws=tab + 16) == ALIAS
    assert mom(geom=(2, 240, 0, 8, 4)) == SHAPE
    assert mom(geom=(0, 240, 240, 8, 4), x=None, tab=None, ws=None) == OK


def _block_weights(C=640, G=32, heads=10, base=A):
    w = dp.BlockWeights(C, G, heads, 1e-5, 0.125)
    for k, name in enumerate(("gn1_gamma", "gn1_beta", "conv_w", "conv_b", "gn2_gamma", "gn2_beta",
                              "w_qkv", "b_qkv", "w_o", "b_o")):
        setattr(w, name, base + k * 64 * MB)
    return w


def _block_state(base):
    s = dp.BlockState()
    for k, name in enumerate(("gn1", "conv_in", "gn2", "k", "v")):
        setattr(s, name, base + k * 1024 * MB)
    return s


def test_block_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    w = _block_weights()
    sin, sout = _block_state(A + (1 << 40)), _block_state(A + (2 << 40))
    x, y, ws = A + (3 << 40), A + (4 << 40), A + (5 << 40)
    n = ctypes.c_size_t(0)
    assert lib.distri_patch_block_workspace_size(G(*g), ctypes.byref(w), BF16, ctypes.byref(n)) == OK
    ns = ctypes.c_size_t(0)
    assert lib.distri_patch_block_sync_workspace_size(G(*g), ctypes.byref(w), BF16,
                                                      ctypes.byref(ns)) == OK
    assert ns.value > 4 * 2 * 240 * 240 * 640 * 2 > n.value > 5 * 2 * 30 * 240 * 640 * 2

    def call(geom=g, w=w, dtype=BF16, x=x, y=y, sin=sin, sout=sout, ws=ws, wsb=None):
        return lib.distri_patch_block(G(*geom), ctypes.byref(w) if w is not None else None, dtype, x,
                                      y, ctypes.byref(sin) if sin is not None else None,
                                      ctypes.byref(sout), ws, n.value if wsb is None else wsb, None)

    assert call(w=None) == NULL
    assert call(w=_block_weights(C=640, heads=8)) == SHAPE      # C != heads * 64
    assert call(w=_block_weights(C=640, G=48)) == SHAPE         # C % G
    assert call(dtype=4) == DTYPE
    assert call(geom=(2, 240, 240, 7, 0)) == SHAPE
    assert call(sin=None) == NULL
    bad = _block_state(A + (1 << 40))
    bad.k = None
    assert call(sin=bad) == NULL
    assert call(wsb=n.value - 1) == WS
    assert call(x=x + 8) == ALIGN
    w2 = _block_weights()
    w2.eps = -1.0
    assert call(w=w2) == SHAPE
    w2 = _block_weights()
    w2.scale = 0.0
    assert call(w=w2) == SHAPE
    w2 = _block_weights()
    w2.w_o = None
    assert call(w=w2) == NULL
    assert call(y=x + 1024) == ALIAS                           # y inside x
    assert call(ws=sin.k + 64) == ALIAS                         # workspace inside a stale map
    part = _block_state(A + (2 << 40))
    part.v = sin.v + 1024                                       # out map overlaps, not equal
    assert call(sout=part) == ALIAS
    part = _block_state(A + (2 << 40))
    part.k = sin.v                                              # out k is in v: different field
    assert call(sout=part) == ALIAS
    assert call(geom=(0, 240, 240, 8, 4), x=None, y=None) == OK

    def sync(wsb=ns.value, st=sout, x=x, y=y):
        return lib.distri_patch_block_sync(G(*g), ctypes.byref(w), BF16, x, y, ctypes.byref(st),
                                           ws, wsb, None)
    assert sync(wsb=ns.value - 1) == WS
    assert sync(y=x + 16) == ALIAS
    same = _block_state(A + (2 << 40))
    same.gn2 = same.gn1
    assert sync(st=same) == ALIAS


def test_cross_attention_rejects_bad_arguments(lib):
    g = (2, 240, 240, 8, 4)
    q, k, v, o = (A + j * 64 * MB for j in range(4))

    def call(geom=g, heads=10, hd=64, ctx=77, scale=0.125, dtype=BF16, q=q, k=k, v=v, o=o, ws=None,
             wsb=0):
        return lib.distri_patch_cross_attn(G(*geom), heads, hd, ctx, scale, dtype, q, k, v, o, ws, wsb,
                                           None)

    assert call(ctx=0) == SHAPE
    assert call(hd=32) == UNSUP
    assert call(heads=0) == SHAPE
    assert call(scale=-1.0) == SHAPE
    assert call(dtype=2) == DTYPE
    assert call(k=None) == NULL
    assert call(v=v + 4) == ALIGN
    assert call(o=k + 64) == ALIAS
    assert call(geom=(0, 240, 240, 8, 4), q=None, k=None, v=None, o=None) == OK
    n = ctypes.c_size_t(0)
    assert lib.distri_patch_cross_attn_workspace_size(G(*g), 10, 64, 77, BF16, ctypes.byref(n)) == OK
    assert lib.distri_patch_cross_attn_workspace_size(G(*g), 10, 64, 0, BF16, ctypes.byref(n)) == SHAPE
    # bf16 contexts of at most 128 tokens are held on chip whole: no workspace
    for ctx in (1, 77, 128):
        n.value = 12345
        assert lib.distri_patch_cross_attn_workspace_size(G(*g), 10, 64, ctx, BF16, ctypes.byref(n)) == OK
        assert n.value == 0


def test_groupnorm_noalloc_rejects_before_any_hip_call(lib):
    """The allocation-free GroupNorm: the same argument checks, and a shape
    whose scratch need exceeds its 2 MiB array is refused (UNSUPPORTED)."""
    def call(geom, C=640, G=32, dtype=BF16, ptrs=None):
        p = ptrs or [A + k * 64 * MB for k in range(6)]
        return lib.distri_async_groupnorm_noalloc(G_(*geom), C, G, 1e-5, dtype, *p, None)
    G_ = G
    assert call((2, 64, 64, 8, 9)) == SHAPE
    assert call((2, 64, 64, 8, 3), C=650) == SHAPE                # C % G != 0
    assert call((2, 64, 64, 8, 3), dtype=9) == DTYPE
    p = [A + k * 64 * MB for k in range(6)]
    p[0] = None
    assert call((2, 64, 64, 8, 3), ptrs=p) == NULL
    p = [A + k * 64 * MB for k in range(6)]
    p[4] = p[0] + 64                                            # y inside x_fresh
    assert call((2, 64, 64, 8, 3), ptrs=p) == ALIAS
    big = (4096, 8, 8, 1, 0)                                    # B * C * 8 bytes of affine alone: 32 MiB
    assert dp.distri_async_groupnorm_workspace_size(big, 1024, 256, BF16) > 2 * MB
    assert call(big, C=1024, G=256) == UNSUP
    assert b"2 MiB" in lib.distri_last_error()
    assert dp.distri_async_groupnorm_workspace_size((2, 240, 240, 8, 4), 640, 32, BF16) < 2 * MB
