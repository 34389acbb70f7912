"""Helpers shared by the GPU parity tests: seeded inputs on both sides,
oracle references, and the tolerance rule.

Tolerance (written once, used by every parity test).  With x the oracle
output (fp64) and y the kernel output in the output dtype, over the whole
output tensor (or the sampled rows of a full-size case):

    max |y - x| <= tol * RMS(x)
    tol = 2e-2 for bf16 inputs (fp32 accumulation), 1e-4 for fp32 inputs

The bound includes the output's own rounding to its dtype.  Each case first
computes, from the oracle alone, its rounding floor F = max |rnd(x) - x| /
RMS(x), rnd = round to nearest even in the output dtype: the score of the
best output that dtype can hold.  Heavy-tailed outputs spend most of the
bound on it (attention: F = 0.017-0.019).  Where F <= tol the bound above is
the rule, unchanged.  Where F > tol no output in that dtype can meet it (the
SiLU form of GroupNorm: F = 0.026; short-context cross-attention: F up to
0.022); there every element must lie within the bound or be the correctly
rounded value of x:

    |y - x| <= max(tol * RMS(x), half_ulp(x) + 2^-12 |x|)  for every element

(2^-12 |x| admits the other neighbour when x lies that close to a rounding
midpoint, the size of the kernels' own arithmetic error).  Each comparison
prints max|y - x| / RMS and F, and appends them to $PARITY_REPORT when that is
set.
  GroupNorm fresh moments: |d m1| <= 1e-5 sqrt(m2) + 1e-7, |d m2| <= 1e-5 m2 + 1e-7
  refresh: bitwise.
"""
from __future__ import annotations

import functools
import json
import os

import numpy as np
import torch

import oracle
import synthetic_inputs as si

TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel_max_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def half_ulp(x, dtype):
    """Half a unit in the last place of |x| in the output dtype (0 at x = 0)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)                  # a = m 2^e, m in [0.5, 1)
    bits = 8 if dtype == "bf16" else 24  # significand bits incl. the implicit one
    return np.where(a > 0, np.ldexp(1.0, e - 1 - bits), 0.0)


def rounding_floor(ref, dtype):
    """max |rnd(x) - x| / RMS(x): the score of the correctly rounded output."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-30)
    return float(np.max(np.abs(oracle.round_to(ref, dtype) - ref))) / rms


def assert_close(got, ref, dtype, what):
    """The parity rule above; returns max|got - ref| / RMS(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-30)
    tol = TOL[dtype]
    err = np.abs(got - ref)
    rel = float(err.max()) / rms
    floor = rounding_floor(ref, dtype)
    print(f"parity {what}: max|err|/RMS = {rel:.4e} (bound {tol:.0e}; rounding floor {floor:.4e})",
          flush=True)
    report = os.environ.get("PARITY_REPORT")
    if report:
        with open(report, "a") as f:
            f.write(json.dumps({"case": what, "dtype": dtype, "max_err_over_rms": rel, "bound": tol,
                                "rounding_floor": floor, "n": int(err.size)}) + "\n")
    if floor <= tol:
        worst = np.unravel_index(int(np.argmax(err)), err.shape)
        assert rel <= tol, (f"{what}: max|err| = {rel:.4e} x RMS exceeds {tol} x RMS at {worst}: "
                            f"got {got[worst]}, oracle {ref[worst]}")
    else:
        allow = np.maximum(tol * rms, half_ulp(ref, dtype) + np.ldexp(np.abs(ref), -12))
        excess = err - allow
        worst = np.unravel_index(int(np.argmax(excess)), err.shape)
        assert excess[worst] <= 0, (f"{what}: rounding floor {floor:.4e} > {tol}, and the element at "
                                    f"{worst} is neither within {tol} x RMS nor correctly rounded: "
                                    f"got {got[worst]}, oracle {ref[worst]}")
    return rel


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


@functools.lru_cache(maxsize=3)
def cpu_inputs(wl: si.Workload, stale_equals_fresh=False):
    d = si.make_inputs(wl, stale_equals_fresh=stale_equals_fresh, nonzero_bias=True)
    # previous step's per-patch moments of the stale map, stored fp32
    table = np.zeros((wl.batch, wl.n_patches, wl.groups, 2))
    for j in range(wl.n_patches):
        table[:, j] = oracle.group_moments(d["x_stale"][:, j * wl.h:(j + 1) * wl.h], wl.groups)
    d["table"] = torch.from_numpy(table).float()
    return d


def gpu_copy(d, dev="cuda"):
    return {k: v.to(dev) for k, v in d.items()}


def sample_rows(total, tile, count=4):
    """Row ranges that cover the first rows, a tile boundary, and the ragged
    tail of [0, total)."""
    ranges = [(0, min(count, total))]
    if total > 2 * tile:
        ranges.append((tile - count // 2, tile + count // 2))
    ranges.append((max(total - count, 0), total))
    out = []
    for r in ranges:
        if r not in out and r[0] < r[1]:
            out.append(r)
    return out
