"""Benchmark of one device's share of a DistriFusion patch layer on MI355X.

A step is one pass of the whole hot path for the 3840^2 SDXL workload split
into n = 8 row patches (this device holds patch 4, an interior patch with both
halos), for both of its UNet feature-map levels:
  (a) 2 x 640 ch x 240 x 240  (57600 tokens, 10 heads x 64, 7200 local queries)
  (b) 2 x 1280 ch x 120 x 120 (14400 tokens, 20 heads x 64, 1800 local queries)
Per level: corrected async GroupNorm -> 3x3 conv with stale halo (its input
is the GroupNorm output) -> self-attention over fresh + stale K/V -> refresh
of K, V, the conv input and the GroupNorm moments into the stale buffers.
Inputs are seeded synthetic bf16 tensors already resident in HBM.

Prints one JSON line.  `value` is (attention + conv FLOPs of both levels) /
step time in TFLOP/s; the step is captured once in a HIP graph and the
timed steps are graph replays (the eager step time is reported beside it).  Per-op figures (attention and conv TFLOP/s, GroupNorm
and refresh GB/s with buffers rotated through > 512 MB so the 256 MB
Infinity Cache cannot serve them) ride along, plus the roofline of the
dominant kernel (attention at level a) and the CPU oracle's rate on a bounded
sample of the same workload.  Reported beside them, outside the step: the
attention layer's Q/K/V (with the fused K/V refresh) and output projections
in TFLOP/s, one asynchronous step of the chained patch block (GroupNorm+SiLU,
halo conv, GroupNorm, projections, attention) and its synchronous warm-up
step over all n patches; cross-attention of the patch queries over a 77-token
context; and the naive-patch layer (each op on this patch alone) for
comparison.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "patch-layer TFLOP/s (attn+conv), GroupNorm GB/s, ms/layer at 3840² n=8"
LEVELS = ("sdxl3840_l2", "sdxl3840_l3")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--patch", type=int, default=4)
    ap.add_argument("--op-iters", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=14.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step with eager launches only (default: also capture it in a "
                         "HIP graph and take the replay time as the step time)")
    ap.add_argument("--profile-op", choices=["attn", "conv", "gn", "refresh", "copy"],
                    help="run only this op (--steps times) for counter collection, print nothing else")
    ap.add_argument("--level", default="sdxl3840_l2", choices=list(LEVELS))
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown table of a rocprofv3 --kernel-trace run under DIR "
                         "(library kernels grouped by name and grid) and exit; needs no GPU")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print per-kernel means of every rocprofv3 --pmc run under DIR and exit")
    return ap.parse_args()


class Level:
    """Device buffers of one workload level (patch `patch`)."""

    def __init__(self, name, patch, dev):
        import torch

        import displaced_patch_parallelism_distri_amd as dp
        import synthetic_inputs as si

        self.wl = wl = si.WORKLOADS[name].with_patch(patch)
        self.geom = wl.geom
        d = si.make_inputs(wl, device=dev, nonzero_bias=True)
        self.t = d
        B, n, G, C = wl.batch, wl.n_patches, wl.groups, wl.channels
        # the previous step's per-patch GroupNorm moments: run the op on every
        # stale patch and refresh each result into the table
        self.table = torch.zeros(B, n, G, 2, dtype=torch.float32, device=dev)
        scratch_table = torch.zeros_like(self.table)
        for j in range(n):
            gj = (B, wl.height, wl.width, n, j)
            xs_j = d["x_stale"][:, j * wl.h:(j + 1) * wl.h].contiguous()
            _, fm = dp.distri_async_groupnorm(gj, G, xs_j, scratch_table, d["gamma"], d["beta"])
            dp.distri_refresh_stale((B, n, 1, n, j), 2 * G, fm, self.table)
        self.conv_stale = d["x_stale"]          # stale conv input map (GN output of last step)
        self.y_gn = torch.empty_like(d["x_fresh"])
        self.fm = torch.empty(B, G, 2, dtype=torch.float32, device=dev)
        code = dp.DISTRI_BF16 if wl.dtype == "bf16" else dp.DISTRI_F32
        self.y_conv = torch.empty(B, wl.h, wl.width, C, dtype=d["x_fresh"].dtype, device=dev)
        self.out = torch.empty_like(d["q"])
        self.gn_ws = torch.empty(dp.distri_async_groupnorm_workspace_size(self.geom, C, G, code),
                                 dtype=torch.uint8, device=dev)
        nb = dp.distri_patch_self_attn_workspace_size(self.geom, wl.heads, 64, code)
        self.attn_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        self.tok_row = wl.width * wl.heads * wl.head_dim
        self.scale = wl.head_dim ** -0.5

    # the individual ops -------------------------------------------------
    def groupnorm(self, x=None, y=None):
        import displaced_patch_parallelism_distri_amd as dp

        dp.distri_async_groupnorm(self.geom, self.wl.groups, self.t["x_fresh"] if x is None else x,
                                  self.table, self.t["gamma"], self.t["beta"], eps=self.wl.eps,
                                  y=self.y_gn if y is None else y, fresh_moments=self.fm,
                                  workspace=self.gn_ws)

    def conv(self):
        import displaced_patch_parallelism_distri_amd as dp

        dp.distri_patch_conv3x3_halo(self.geom, self.y_gn, self.conv_stale, self.t["weight"],
                                     self.t["bias"], y=self.y_conv)

    def attention(self):
        import displaced_patch_parallelism_distri_amd as dp

        t = self.t
        dp.distri_patch_self_attn(self.geom, self.wl.heads, t["q"], t["k_fresh"], t["v_fresh"],
                                  t["k_stale"], t["v_stale"], out=self.out, scale=self.scale,
                                  workspace=self.attn_ws)

    def refresh_maps(self, k=None, v=None, x=None, fm=None, ks=None, vs=None, xs=None, tab=None):
        """The layer's four stale maps (K, V, conv input, moment table) as
        (rows, row_elems, fresh, stale) for distri_refresh_stale_maps."""
        t, wl = self.t, self.wl
        pick = lambda a, b: b if a is None else a
        return [(wl.h, self.tok_row, pick(k, t["k_fresh"]), pick(ks, t["k_stale"])),
                (wl.h, self.tok_row, pick(v, t["v_fresh"]), pick(vs, t["v_stale"])),
                (wl.h, wl.width * wl.channels, pick(x, self.y_gn), pick(xs, self.conv_stale)),
                (1, 2 * wl.groups, pick(fm, self.fm), pick(tab, self.table))]

    def refresh(self):
        import displaced_patch_parallelism_distri_amd as dp

        dp.distri_refresh_stale_maps(self.geom, self.refresh_maps())

    def layer(self, ev=None):
        self.groupnorm()
        self.conv()
        if ev is not None:
            ev[0].record()
        self.attention()
        if ev is not None:
            ev[1].record()
        self.refresh()


def time_op(fn, iters, warmup=3, reps=1):
    """Median and minimum per-call time (ms) over `iters` samples; a sample
    is `reps` back-to-back calls between two events, so for the short
    memory-bound ops the event overhead is amortised while the gaps between
    consecutive launches still count."""
    import torch

    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    k = 0
    for a, b in evs:
        a.record()
        for _ in range(reps):
            k += 1
            fn(k)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) / reps for a, b in evs)
    return ts[len(ts) // 2], ts[0]


def per_op(levels, iters):
    """Median per-op times; GroupNorm and refresh rotate through > 512 MB."""
    import torch

    res = {}
    for lv in levels:
        wl = lv.wl
        key = wl.name
        slice_bytes = wl.slice_bytes()
        nrot = max(2, int(math.ceil(600e6 / (2 * slice_bytes))))
        xs = [torch.randn_like(lv.t["x_fresh"], dtype=torch.float32).to(torch.bfloat16) for _ in range(nrot)]
        ys = [torch.empty_like(lv.t["x_fresh"]) for _ in range(nrot)]
        gn_med, gn_min = time_op(lambda k: lv.groupnorm(xs[k % nrot], ys[k % nrot]), iters, reps=10)
        del xs, ys
        # the layer's refresh, all four maps in one call (K, V, conv input,
        # moment table), rotating through sets of fresh slices and stale maps
        # (the contents do not matter for a bitwise copy)
        import displaced_patch_parallelism_distri_amd as dp

        t = lv.t
        sets = []
        for _ in range(3):
            e = lambda a: torch.empty_like(a)
            sets.append(lv.refresh_maps(k=e(t["k_fresh"]), v=e(t["v_fresh"]), x=e(t["x_fresh"]), fm=e(lv.fm),
                                        ks=e(t["k_stale"]), vs=e(t["v_stale"]), xs=e(lv.conv_stale),
                                        tab=e(lv.table)))
        refresh_bytes = sum(m[2].numel() * m[2].element_size() for m in sets[0])
        rf_med, rf_min = time_op(lambda k: dp.distri_refresh_stale_maps(lv.geom, sets[k % 3]), iters, reps=10)
        del sets
        cv_med, cv_min = time_op(lambda k: lv.conv(), iters)
        at_med, at_min = time_op(lambda k: lv.attention(), iters)
        res[key] = {
            "groupnorm_ms": gn_med, "groupnorm_gbps": 2 * slice_bytes / gn_med / 1e6,
            "refresh_ms": rf_med, "refresh_gbps": 2 * refresh_bytes / rf_med / 1e6,
            "refresh_bytes_read": refresh_bytes,
            "conv_ms": cv_med, "conv_tflops": wl.conv_flops() / cv_med / 1e9,
            "attention_ms": at_med, "attention_tflops": wl.attn_flops() / at_med / 1e9,
        }
        torch.cuda.empty_cache()
    return res


def block_bench(levels, iters):
    """The attention layer's projections and the chained patch block at each
    level (outside the step above): Q/K/V projection with its fused K/V
    refresh and the output projection in TFLOP/s, one asynchronous block step
    of this patch, and the synchronous warm-up step of all n patches."""
    import torch

    import displaced_patch_parallelism_distri_amd as dp
    import synthetic_inputs as si

    res = {}
    for lv in levels:
        wl = lv.wl
        B, C, n, h, Lq = wl.batch, wl.channels, wl.n_patches, wl.h, wl.lq
        M = B * Lq
        d = si.make_block_inputs(wl, device="cuda")
        w, st = d["weights"], d["state"]
        x = d["x"][:, wl.patch * h:(wl.patch + 1) * h].contiguous()
        xq = x.view(B, Lq, C)
        q, k, v, o = (torch.empty(B, Lq, C, dtype=torch.bfloat16, device="cuda") for _ in range(4))
        y = torch.empty_like(q)
        # the short ops are timed 10 back-to-back calls per sample (as the
        # memory-bound ops are), which amortises the event overhead
        qkv_ms, _ = time_op(lambda i: dp.distri_patch_qkv_proj(wl.geom, xq, w["w_qkv"], w["b_qkv"], q, k, v,
                                                               st["k"], st["v"]), iters, reps=10)
        out_ms, _ = time_op(lambda i: dp.distri_patch_out_proj(wl.geom, xq, w["w_o"], w["b_o"], o), iters,
                            reps=10)
        kw = dict(groups=wl.groups, heads=wl.heads, eps=wl.eps, scale=wl.head_dim ** -0.5)
        ws = torch.empty(dp.distri_patch_block_workspace_size(wl.geom, C, wl.groups, wl.heads,
                                                              dp.DISTRI_BF16), dtype=torch.uint8,
                         device="cuda")
        blk_ms, _ = time_op(lambda i: dp.distri_patch_block(wl.geom, w, x, st, y=y, workspace=ws, **kw),
                            iters)
        del ws
        xp = d["x"].view(B, n, h, wl.width, C).transpose(0, 1).contiguous()
        ys = torch.empty(n, B, Lq, C, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(dp.distri_patch_block_sync_workspace_size(wl.geom, C, wl.groups, wl.heads,
                                                                   dp.DISTRI_BF16), dtype=torch.uint8,
                         device="cuda")
        sync_ms, _ = time_op(lambda i: dp.distri_patch_block_sync(wl.geom, w, xp, st, y=ys, workspace=ws,
                                                                  **kw), max(5, iters // 4))
        # cross-attention of the patch queries over a 77-token context, and
        # the naive-patch layer (each op on this patch alone)
        cx = si.make_cross_inputs(wl, 77, device="cuda")
        co = torch.empty_like(cx["q"])
        cws = torch.empty(max(1, dp.distri_patch_cross_attn_workspace_size(wl.geom, wl.heads, 77,
                                                                           dp.DISTRI_BF16)),
                          dtype=torch.uint8, device="cuda")
        cx_ms, _ = time_op(lambda i: dp.distri_patch_cross_attn(wl.geom, wl.heads, cx["q"], cx["k_ctx"],
                                                                cx["v_ctx"], out=co, workspace=cws), iters,
                            reps=10)
        cx_bytes = 2 * (2 * cx["q"].numel() + 2 * cx["k_ctx"].numel())  # Q, O, context K and V
        cx_fl = 4.0 * B * wl.heads * Lq * 77 * wl.head_dim
        del cx, co, cws
        ng = dp.naive_geom(wl.geom)
        t = lv.t
        zt = torch.zeros(B, 1, wl.groups, 2, device="cuda")

        def naive_layer(i):
            yg, _ = dp.distri_async_groupnorm(ng, wl.groups, t["x_fresh"], zt, t["gamma"], t["beta"])
            dp.distri_patch_conv3x3_halo(ng, yg, None, t["weight"], t["bias"])
            dp.distri_patch_self_attn(ng, wl.heads, t["q"], t["k_fresh"], t["v_fresh"], t["k_fresh"],
                                      t["v_fresh"])
        naive_ms, _ = time_op(naive_layer, iters)
        qkv_fl, out_fl = 2.0 * M * 3 * C * C, 2.0 * M * C * C
        blk_fl = wl.attn_flops() + wl.conv_flops() + qkv_fl + out_fl
        res[wl.name] = {
            "qkv_proj_ms": qkv_ms, "qkv_proj_tflops": qkv_fl / qkv_ms / 1e9,
            "out_proj_ms": out_ms, "out_proj_tflops": out_fl / out_ms / 1e9,
            "block_async_ms": blk_ms, "block_async_tflops": blk_fl / blk_ms / 1e9,
            "block_sync_all_patches_ms": sync_ms,
            "cross_attn_ctx77_ms": cx_ms, "cross_attn_ctx77_tflops": cx_fl / cx_ms / 1e9,
            "cross_attn_ctx77_gbps": cx_bytes / cx_ms / 1e6,
            "naive_patch_layer_ms": naive_ms,
        }
        del d, w, st, x, xp, ys, ws, q, k, v, o, y
        torch.cuda.empty_cache()
    return res


def copy_peak(iters):
    """Achievable HBM rate of a large copy (read + write bytes / time): the
    library's refresh kernel over a whole 512 MiB map (n = 1) and torch's
    device copy of the same buffers."""
    import torch

    import displaced_patch_parallelism_distri_amd as dp

    nbytes = 512 << 20
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    rows = 1024
    geom = (1, rows, 1, 1, 0)
    rf, _ = time_op(lambda k: dp.distri_refresh_stale(geom, nbytes // 2 // rows, src, dst), iters)
    rm, _ = time_op(lambda k: dp.distri_refresh_stale_maps(geom, [(rows, nbytes // 2 // rows, src, dst)]),
                    iters)
    tc, _ = time_op(lambda k: dst.copy_(src), iters)
    del src, dst
    torch.cuda.empty_cache()
    return {"refresh_kernel_gbps": round(2 * nbytes / rf / 1e6, 1),
            "refresh_maps_kernel_gbps": round(2 * nbytes / rm / 1e6, 1),
            "torch_copy_gbps": round(2 * nbytes / tc / 1e6, 1), "bytes_copied": nbytes}


def cpu_baseline(budget_s):
    """The CPU oracle on a bounded sample of level (a): the first local query
    rows of attention (both images, all 10 heads, all 57600 keys) and the
    first output row of the conv.  Inputs are widened to float64 before the
    clock starts; the rate is (sample FLOPs) / (oracle wall time)."""
    import numpy as np

    import oracle
    import synthetic_inputs as si

    wl = si.WORKLOADS["sdxl3840_l2"].with_patch(4)
    d = si.make_inputs(wl, device="cpu", nonzero_bias=True)
    f64 = {k: np.ascontiguousarray(v.double().numpy()) for k, v in d.items()}
    del d
    scale = wl.head_dim ** -0.5
    args = (f64["q"], f64["k_fresh"], f64["v_fresh"], f64["k_stale"], f64["v_stale"])
    t0 = time.perf_counter()
    oracle.patch_self_attn(wl.geom, wl.heads, 64, scale, *args, rows=(0, 16))
    per_row = (time.perf_counter() - t0) / 16
    rows = int(max(16, min(wl.lq, 0.85 * budget_s / max(per_row, 1e-6))))
    t0 = time.perf_counter()
    oracle.patch_self_attn(wl.geom, wl.heads, 64, scale, *args, rows=(0, rows))
    ta = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, f64["x_fresh"], f64["x_stale"],
                              f64["weight"], f64["bias"], rows=(0, 1))
    tc = time.perf_counter() - t0
    fa = 4.0 * wl.batch * wl.heads * rows * wl.tokens * wl.head_dim
    fc = 2.0 * wl.batch * wl.width * wl.channels * wl.channels * 9
    return {"value": (fa + fc) / (ta + tc) / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"sdxl3840 level (a) patch 4, fp64: attention for {rows} local query rows x 2 "
                      f"images x 10 heads over 57600 keys + conv for 1 output row (2 x 240 px x "
                      f"640 -> 640 ch); {ta + tc:.1f} s of oracle time",
            "seconds": round(ta + tc, 2)}


SMALL_CONFIGS = ("tiny", "sdxl1024_l2", "sdxl1024_l3")


def _small_patch(wl):
    return wl.n_patches // 2


def oracle_one_core():
    """The oracle's time per op on one host core (its OpenMP thread count set
    to 1 for these calls, then restored) on the three small configurations,
    interior patch.  Attention runs on the first min(Lq, 64) local query
    rows and the conv on one output row; both are scaled to the whole patch
    by the row count (their cost is linear in it).  GroupNorm runs whole."""
    import numpy as np

    import oracle
    import synthetic_inputs as si

    before = oracle.num_threads()
    oracle.set_num_threads(1)
    res = {"threads": oracle.num_threads()}
    for name in SMALL_CONFIGS:
        base = si.WORKLOADS[name]
        wl = base.with_patch(_small_patch(base))
        d = si.make_inputs(wl, device="cpu", nonzero_bias=True)
        f = {k: np.ascontiguousarray(v.double().numpy()) for k, v in d.items()}
        B, n, G, h = wl.batch, wl.n_patches, wl.groups, wl.h
        table = np.zeros((B, n, G, 2))
        for j in range(n):
            table[:, j] = oracle.group_moments(f["x_stale"][:, j * h:(j + 1) * h], G)
        ra = min(wl.lq, 64)
        t0 = time.perf_counter()
        oracle.patch_self_attn(wl.geom, wl.heads, 64, wl.head_dim ** -0.5, f["q"], f["k_fresh"], f["v_fresh"],
                               f["k_stale"], f["v_stale"], rows=(0, ra))
        ta = (time.perf_counter() - t0) * wl.lq / ra
        t0 = time.perf_counter()
        oracle.patch_conv3x3_halo(wl.geom, wl.channels, wl.channels, f["x_fresh"], f["x_stale"], f["weight"],
                                  f["bias"], rows=(0, 1))
        tc = (time.perf_counter() - t0) * h
        t0 = time.perf_counter()
        oracle.async_groupnorm(wl.geom, wl.channels, G, wl.eps, f["x_fresh"], table, f["gamma"], f["beta"])
        tg = time.perf_counter() - t0
        res[name] = {"attention_ms": ta * 1e3, "conv_ms": tc * 1e3, "groupnorm_ms": tg * 1e3,
                     "sample": f"patch {wl.patch} of {n}; attention {ra} of {wl.lq} query rows and conv "
                               f"1 of {h} output rows, scaled by the row count; GroupNorm whole"}
    oracle.set_num_threads(before)
    return res


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def small_config_comparison(iters):
    """The oracle on one host core against the kernels on the GPU, per op,
    on the three small configurations."""
    import torch

    cpu = oracle_one_core()
    dev = torch.device("cuda:0")
    out = {"oracle_threads": cpu.pop("threads")}
    for name in SMALL_CONFIGS:
        base = __import__("synthetic_inputs").WORKLOADS[name]
        lv = Level(name, _small_patch(base), dev)
        gpu = {"attention_ms": time_op(lambda k: lv.attention(), iters)[0],
               "conv_ms": time_op(lambda k: lv.conv(), iters)[0],
               "groupnorm_ms": time_op(lambda k: lv.groupnorm(), iters, reps=10)[0]}
        row = {"dtype": lv.wl.dtype, "sample": cpu[name]["sample"]}
        for op in ("attention", "conv", "groupnorm"):
            c, g = cpu[name][op + "_ms"], gpu[op + "_ms"]
            row[op] = {"oracle_1core_ms": round(c, 3), "gpu_ms": round(g, 4), "speedup": round(c / g, 1)}
        out[name] = row
        del lv
    torch.cuda.empty_cache()
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_sdxl3840_traffic_counters.md")
ATTN_SRC = os.path.join(ROOT, "displaced_patch_parallelism_distri_amd", "csrc", "attention.hip")


def measured_traffic():
    """HBM bytes per launch of the level-(a) attention kernel from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None when the
    kernel source changed since those counters were taken."""
    import hashlib

    try:
        text = open(TRAFFIC_FILE).read()
        src = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith(("source_sha256", "traffic_bytes_per_launch")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != src or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def profile_op(args):
    """Run one op --steps times (for rocprofv3 counter runs)."""
    import torch

    lv = Level(args.level, args.patch, torch.device("cuda:0"))
    if args.profile_op == "copy":
        # plain device copy of known size, to calibrate FETCH_SIZE/WRITE_SIZE
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
    else:
        fn = {"attn": lv.attention, "conv": lv.conv, "gn": lv.groupnorm, "refresh": lv.refresh}[args.profile_op]
    torch.cuda.synchronize()
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()


def _short_kernel(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].replace("unsigned int __vector", "u32x4")


def summarize_trace(d):
    """Per (kernel, grid) launch count and mean/min/max duration in us, from
    rocprofv3's kernel trace csv."""
    import collections
    import csv
    import glob

    path = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if "dp::" not in r["Kernel_Name"]:
            continue
        grid = "%sx%sx%s / %s" % (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"], r["Workgroup_Size_X"])
        agg[(_short_kernel(r["Kernel_Name"]), grid, r["VGPR_Count"], r["Accum_VGPR_Count"],
             r["LDS_Block_Size"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | grid (threads) / block | VGPR | AGPR | LDS B | calls | mean us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|---|")
    for (k, g, v, a, l), t in sorted(agg.items()):
        print(f"| {k} | {g} | {v} | {a} | {l} | {len(t)} | {sum(t) / len(t):.2f} | {min(t):.2f} | {max(t):.2f} |")


def summarize_counters(d):
    """Per (run, kernel, counter) mean over dispatches, from rocprofv3's
    counter collection csv files."""
    import collections
    import csv
    import glob

    print("| run | kernel | counter | dispatches | mean |")
    print("|---|---|---|---|---|")
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        run = os.path.relpath(os.path.dirname(path), d)
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            k = _short_kernel(r["Kernel_Name"])
            if k.startswith("dp::") or "copyBuffer" in k:
                agg[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
        for (k, c), v in sorted(agg.items()):
            print(f"| {run} | {k} | {c} | {len(v)} | {sum(v) / len(v):.1f} |")


def main():
    args = parse()
    if args.summarize_trace or args.summarize_counters:
        if args.summarize_trace:
            summarize_trace(args.summarize_trace)
        if args.summarize_counters:
            summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the exchange between patch devices is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    import displaced_patch_parallelism_distri_amd as dp

    dp.load()
    if args.profile_op:
        profile_op(args)
        return
    dev = torch.device("cuda:0")
    levels = [Level(n, args.patch, dev) for n in LEVELS]
    torch.cuda.synchronize()

    # whole-step timing
    for _ in range(args.warmup):
        for lv in levels:
            lv.layer()
    torch.cuda.synchronize()
    attn_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    layer_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        layer_ev[k][0].record()
        levels[0].layer(attn_ev[k])
        layer_ev[k][1].record()
        levels[1].layer()
        layer_ev[k][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps
    la = sorted(e[0].elapsed_time(e[1]) for e in layer_ev)
    lb = sorted(e[1].elapsed_time(e[2]) for e in layer_ev)
    attn_ms = sum(a.elapsed_time(b) for a, b in attn_ev) / args.steps

    # the same step captured once in a HIP graph and replayed: the launch
    # gaps between the step's 20 kernels shrink to the graph's
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for lv in levels:
                lv.layer()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for lv in levels:
                lv.layer()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del g

    flops = sum(lv.wl.attn_flops() + lv.wl.conv_flops() for lv in levels)
    eager_ms = step_ms
    if graph_ms is not None:
        step_ms = graph_ms
    value = flops / (step_ms * 1e-3) / 1e12
    ops = per_op(levels, args.op_iters)
    copy = copy_peak(args.op_iters)
    blocks = block_bench(levels, args.op_iters)

    wa = levels[0].wl
    achieved = wa.attn_flops() / (attn_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_eager": round(eager_ms, 4),
        "step_launch": "hip graph replay" if graph_ms is not None else "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations of SDXL feature-map shape; no weights, no COCO)",
        "config": {"workload": "sdxl3840 n=8 patch %d: (a) 2x640x240x240 10 heads + (b) 2x1280x120x120 "
                               "20 heads; GN 32 groups, conv 3x3 C->C, attention d=64" % args.patch,
                   "n_patches": 8, "patch": args.patch},
        "ms_per_layer": {"sdxl3840_l2": round(la[len(la) // 2], 4), "sdxl3840_l3": round(lb[len(lb) // 2], 4)},
        "per_op": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in ops.items()},
        "groupnorm_gbps": {k: round(v["groupnorm_gbps"], 1) for k, v in ops.items()},
        "refresh_gbps": {k: round(v["refresh_gbps"], 1) for k, v in ops.items()},
        "hbm_copy_peak": copy,
        "projections_and_block": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in blocks.items()},
        "roofline": {"kernel": "attention at level a (attn_bf16_kernel + attn_combine_kernel)",
                     "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
                     "avg_launch_ms": round(attn_ms, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        out["cpu_baseline"].update(cpu_info())
        out["cpu_baseline"]["small_configs_one_core"] = small_config_comparison(args.op_iters)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
