"""Brute-force pure-Python versions of the patch layer for tiny inputs.

Test-only.  Written independently of the oracle: each builds the full hybrid
map first (stale map, patch i's rows overwritten by the fresh rows) as nested
Python lists, then evaluates the textbook layer on it element by element with
``math`` only.  Inputs are numpy float64 arrays.
"""
from __future__ import annotations

import math


def _hybrid(fresh, stale, lo, hi):
    """Python nested list of ``stale`` along axis 1 with [lo, hi) from fresh."""
    out = stale.tolist()
    f = fresh.tolist()
    for b in range(len(out)):
        for r in range(lo, hi):
            out[b][r] = f[b][r - lo]
    return out


def attention(geom, scale, q, kf, vf, ks, vs):
    B, H, W, n, i = geom
    Lq = (H // n) * W
    K = _hybrid(kf, ks, i * Lq, (i + 1) * Lq)
    V = _hybrid(vf, vs, i * Lq, (i + 1) * Lq)
    Q = q.tolist()
    heads, d = len(Q[0][0]), len(Q[0][0][0])
    L = H * W
    out = [[[[0.0] * d for _ in range(heads)] for _ in range(Lq)] for _ in range(B)]
    for b in range(B):
        for r in range(Lq):
            for hd in range(heads):
                logits = []
                for t in range(L):
                    logits.append(scale * sum(Q[b][r][hd][e] * K[b][t][hd][e] for e in range(d)))
                top = max(logits)
                wts = [math.exp(x - top) for x in logits]
                tot = sum(wts)
                for e in range(d):
                    out[b][r][hd][e] = sum(wts[t] * V[b][t][hd][e] for t in range(L)) / tot
    return out


def conv3x3(geom, xf, xs, w, bias):
    B, H, W, n, i = geom
    h = H // n
    X = _hybrid(xf, xs, i * h, (i + 1) * h)
    Wt = w.tolist()
    cout, cin = len(Wt), len(Wt[0][0][0])
    y = [[[[0.0] * cout for _ in range(W)] for _ in range(h)] for _ in range(B)]
    for b in range(B):
        for r in range(h):
            gr = i * h + r
            for c in range(W):
                for o in range(cout):
                    acc = 0.0 if bias is None else float(bias[o])
                    for kh in range(3):
                        for kw in range(3):
                            rr, cc = gr + kh - 1, c + kw - 1
                            if 0 <= rr < H and 0 <= cc < W:
                                for ci in range(cin):
                                    acc += Wt[o][kh][kw][ci] * X[b][rr][cc][ci]
                    y[b][r][c][o] = acc
    return y


def groupnorm(geom, groups, eps, xf, xs, gamma, beta):
    """GroupNorm over the whole hybrid map, rows of patch i returned."""
    B, H, W, n, i = geom
    h = H // n
    X = _hybrid(xf, xs, i * h, (i + 1) * h)
    C = len(X[0][0][0])
    cg = C // groups
    y = [[[[0.0] * C for _ in range(W)] for _ in range(h)] for _ in range(B)]
    for b in range(B):
        for g in range(groups):
            vals = [X[b][r][c][ch] for r in range(H) for c in range(W) for ch in range(g * cg, (g + 1) * cg)]
            mu = sum(vals) / len(vals)
            var = sum((v - mu) ** 2 for v in vals) / len(vals)
            for r in range(h):
                for c in range(W):
                    for ch in range(g * cg, (g + 1) * cg):
                        ga = 1.0 if gamma is None else float(gamma[ch])
                        be = 0.0 if beta is None else float(beta[ch])
                        y[b][r][c][ch] = (X[b][i * h + r][c][ch] - mu) / math.sqrt(var + eps) * ga + be
    return y
