"""Pure-Python scalar brute force of the PT-DiT attention core, for tiny grids.

Written independently of oracle/: no NumPy in the arithmetic, explicit loops,
and shifted-window attention in its *group form* (each axis of the padded grid
splits into the groups [0, s), [s, s+w), ..., [L-w+s, L); attention runs inside
every product of groups), rather than the roll-and-mask form the oracle uses.
Pad tokens (coordinates past the real grid, up to a multiple of the window)
are zero vectors, so their projections are the biases.

Used only to pin the oracle (tests marked "not gpu").
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence


def _lin(vec: List[float], W, b) -> List[float]:
    # y_o = sum_i W[o][i] * x_i + b_o
    out = []
    for o in range(len(W)):
        acc = 0.0
        row = W[o]
        for i in range(len(vec)):
            acc += row[i] * vec[i]
        out.append(acc + (b[o] if b is not None else 0.0))
    return out


def _attend(qs: List[List[float]], ks: List[List[float]], vs: List[List[float]],
            heads: int) -> List[List[float]]:
    D = len(qs[0])
    dh = D // heads
    scale = 1.0 / math.sqrt(dh)
    outs = []
    for q in qs:
        o = [0.0] * D
        for h in range(heads):
            lo = h * dh
            scores = []
            for k in ks:
                s = 0.0
                for c in range(lo, lo + dh):
                    s += q[c] * k[c]
                scores.append(s * scale)
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            for c in range(lo, lo + dh):
                acc = 0.0
                for j, v in enumerate(vs):
                    acc += e[j] / z * v[c]
                o[c] = acc
        outs.append(o)
    return outs


def mha_set(tokens_q: List[List[float]], tokens_kv: List[List[float]], w: Dict, heads: int):
    qs = [_lin(t, w["wq"], w["bq"]) for t in tokens_q]
    ks = [_lin(t, w["wk"], w["bk"]) for t in tokens_kv]
    vs = [_lin(t, w["wv"], w["bv"]) for t in tokens_kv]
    os_ = _attend(qs, ks, vs, heads)
    return [_lin(o, w["wo"], w["bo"]) for o in os_]


def pool(x, grid, p):
    """x: [N][D] lists for one sample; returns [M][D] exact means (math.fsum)."""
    F, H, W = grid
    D = len(x[0])
    out = []
    for T in range(F // p[0]):
        for I in range(H // p[1]):
            for J in range(W // p[2]):
                members = []
                for dt in range(p[0]):
                    for di in range(p[1]):
                        for dj in range(p[2]):
                            t, i, j = T * p[0] + dt, I * p[1] + di, J * p[2] + dj
                            members.append(x[(t * H + i) * W + j])
                out.append([math.fsum(m[c] for m in members) / len(members) for c in range(D)])
    return out


def _axis_groups(L: int, w: int, s: int) -> List[List[int]]:
    """Groups of one axis of the padded length L for window w, shift s."""
    if s == 0:
        return [list(range(a, a + w)) for a in range(0, L, w)]
    groups = [list(range(0, s))]
    a = s
    while a + w <= L:
        groups.append(list(range(a, a + w)))
        a += w
    if a < L:
        groups.append(list(range(a, L)))
    return groups


def _window_groups(grid, win, shift):
    Lp = [-(-g // w) * w for g, w in zip(grid, win)]
    gt = _axis_groups(Lp[0], win[0], shift[0])
    gh = _axis_groups(Lp[1], win[1], shift[1])
    gw = _axis_groups(Lp[2], win[2], shift[2])
    out = []
    for a in gt:
        for b in gh:
            for c in gw:
                out.append([(t, i, j) for t in a for i in b for j in c])
    return out


def window_attention(x, grid, win, shift, w, heads, residual=True):
    """Window (shift 0) or shifted-window attention in group form, with the
    zero-pad reading; x: [N][D] lists for one sample."""
    F, H, W = grid
    D = len(x[0])
    out = [list(r) for r in x] if residual else [[0.0] * D for _ in x]

    def tok(t, i, j):
        if t < F and i < H and j < W:
            return x[(t * H + i) * W + j]
        return [0.0] * D

    for g in _window_groups(grid, win, shift):
        toks = [tok(*c) for c in g]
        res = mha_set(toks, toks, w, heads)
        for (t, i, j), r in zip(g, res):
            if t < F and i < H and j < W:
                n = (t * H + i) * W + j
                for c in range(D):
                    out[n][c] += r[c]
    return out


def block(x, grid, p, win, shift, weights, heads):
    """x: [B][N][D]; returns x3 as nested lists."""
    outs = []
    for xb in x:
        P = pool(xb, grid, p)
        Pa = mha_set(P, P, weights[0], heads)
        P2 = [[a + b for a, b in zip(r, s)] for r, s in zip(P, Pa)]
        xa = mha_set(xb, P2, weights[1], heads)
        x1 = [[a + b for a, b in zip(r, s)] for r, s in zip(xb, xa)]
        x2 = window_attention(x1, grid, win, (0, 0, 0), weights[2], heads)
        x3 = window_attention(x2, grid, win, shift, weights[3], heads)
        outs.append(x3)
    return outs


def group_sizes(grid, win, shift) -> List[int]:
    return sorted({len(g) for g in _window_groups(grid, win, shift)})
