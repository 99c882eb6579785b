"""Float64 NumPy oracle of the backward pass of the PT-DiT attention core.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests/ and
bench.py's cpu_baseline leg, never by the GPU path.

What is differentiated: the forward maps of ptdit_oracle, which follow the
Qihoo-T2X reading note, section 3 "Method" (Eq. GIIM, Eq. TCM, and the
code-correspondence excerpt of the PT-Block forward). The pages train the
model at 2048^2 (section 4, training details) but print no backward formulas,
so the backward is the exact gradient of those maps (reading R-bwd); the
tests pin it to central finite differences of the forward and to adjoint
identities, never to itself.

Readings (in addition to the forward readings of ptdit_oracle):
  R-bwd      gradients are those of the forward maps as written, in float64;
             with S = Q K^T / sqrt(d_h), A = softmax(S) over the allowed keys
             and O = A V, given dO: dV = A^T dO, dA = dO V^T,
             dS = A * (dA - rowsum(A * dA)), dQ = dS K / sqrt(d_h),
             dK = dS^T Q / sqrt(d_h) (per head).
  R-bwd-pad  TCM's pad tokens are zero tokens before the projections, so
             their keys and values are the biases b_k, b_v: the gradient that
             reaches a pad key or value slot is added to d b_k / d b_v. Pad
             queries are cropped, so they receive no gradient.
  R-bwd-core the backward of the window attention is taken at the attention
             core: from (Q, K, V, dO) of the real tokens to (dQ, dK, dV) and
             the pad-slot sums; the projections' gradients are the linear-map
             gradients of linear_bwd (dX = dY W, dW = dY^T X, db = sum dY).
  R-bwd-block the block's gradient (block_bwd) is that of <x3, dout> with
             respect to x and all 32 weight and bias tensors, through the
             chain of excerpt 2's order: SWSA, WSA, cross-attention, proxy
             self-attention, window average; the residuals pass the gradient
             through unchanged, and P' feeds both the cross-attention's keys
             and values and (through its residual) back into the window
             average's gradient.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .ptdit_oracle import Grid, _f64, _padded, pad_grid, partition, proxy_grid, region_labels, roll3d, unpartition

__all__ = ["attention_bwd", "window_core", "window_core_bwd", "proxy_pool_bwd", "roll3d_bwd", "linear_bwd",
           "mha_bwd", "window_mha_bwd", "block_bwd"]


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, heads: int,
                  allow: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradient of ptdit_oracle.attention (reading R-bwd).

    q, do: [..., Lq, D]; k, v: [..., Lk, D]; allow as in the forward.
    Returns dq [..., Lq, D], dk, dv [..., Lk, D].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    D = q.shape[-1]
    dh = D // heads
    scale = 1.0 / np.sqrt(dh)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        s = (q[..., sl] @ np.swapaxes(k[..., sl], -1, -2)) * scale
        if allow is not None:
            s = np.where(allow, s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=-1, keepdims=True)                     # softmax weights
        dv[..., sl] = np.swapaxes(a, -1, -2) @ do[..., sl]
        da = do[..., sl] @ np.swapaxes(v[..., sl], -1, -2)        # dL/dA
        ds = a * (da - (a * da).sum(axis=-1, keepdims=True))      # softmax Jacobian
        dq[..., sl] = (ds @ k[..., sl]) * scale
        dk[..., sl] = (np.swapaxes(ds, -1, -2) @ q[..., sl]) * scale
    return dq, dk, dv


def _window_layout(B: int, grid: Grid, win: Sequence[int], shift: Sequence[int]):
    """Allow mask [B*nwin, L, L] of the (shifted) windows: no mask without a
    shift (the forward's WSA), region labels with one (reading R-mask)."""
    padded = _padded(grid, win)
    L = int(np.prod(win))
    if not any(shift):
        return None
    lab = partition(region_labels(padded, win, shift)[None, ..., None], win).reshape(-1, L)
    lab = np.broadcast_to(lab, (B,) + lab.shape).reshape(-1, L)
    return lab[:, :, None] == lab[:, None, :]


def _to_windows(t: np.ndarray, grid: Grid, win: Sequence[int], shift: Sequence[int],
                pad_row: Optional[np.ndarray]) -> np.ndarray:
    """Token-major [B, N, D] -> windows [B*nwin, L, D]: pad to the window grid
    (pad tokens = pad_row, reading R-bwd-pad), roll by -s, partition."""
    B, N, D = t.shape
    tp = pad_grid(t, grid, win)
    if pad_row is not None:
        real = np.zeros(tp.shape[1:4], dtype=bool)
        real[:grid[0], :grid[1], :grid[2]] = True
        tp[:, ~real] = _f64(pad_row)
    z = roll3d(tp, shift) if any(shift) else tp
    return partition(z, win).reshape(-1, int(np.prod(win)), D)


def _from_windows(w: np.ndarray, B: int, grid: Grid, win: Sequence[int], shift: Sequence[int]):
    """Inverse of _to_windows: windows -> padded grid (rolled back by +s);
    returns the padded grid [B, F', H', W', D]."""
    padded = _padded(grid, win)
    nwin = [p // s for p, s in zip(padded, win)]
    g = unpartition(w.reshape(B, *nwin, w.shape[1], w.shape[2]), win)
    return roll3d(g, shift, inverse=True) if any(shift) else g


def window_core(q: np.ndarray, k: np.ndarray, v: np.ndarray, grid: Grid, win: Sequence[int],
                shift: Sequence[int], heads: int, kpad: Optional[np.ndarray] = None,
                vpad: Optional[np.ndarray] = None) -> np.ndarray:
    """The attention core of WSA (shift 0) / SWSA (Eq. TCM), on projected
    token-major q, k, v [B, N, D]: pad (pad keys/values = kpad/vpad, the
    biases b_k/b_v; zero when None), roll by -s, attention inside each window
    under the boundary mask, roll back, crop. Returns O [B, N, D]. With
    q/k/v = Lin(x) and kpad/vpad = b_k/b_v, Lin(O; W_o, b_o) is window_sa /
    shift_window_sa without the residual (a test checks this)."""
    B, N, D = _f64(q).shape
    zero = np.zeros(D)
    qw = _to_windows(_f64(q), grid, win, shift, None)
    kw = _to_windows(_f64(k), grid, win, shift, zero if kpad is None else kpad)
    vw = _to_windows(_f64(v), grid, win, shift, zero if vpad is None else vpad)
    from .ptdit_oracle import attention
    ow = attention(qw, kw, vw, heads, _window_layout(B, grid, win, shift))
    og = _from_windows(ow, B, grid, win, shift)
    return og[:, :grid[0], :grid[1], :grid[2]].reshape(B, N, D)


def window_core_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, grid: Grid,
                    win: Sequence[int], shift: Sequence[int], heads: int,
                    kpad: Optional[np.ndarray] = None, vpad: Optional[np.ndarray] = None):
    """Gradient of window_core (readings R-bwd, R-bwd-pad).

    Returns dq, dk, dv [B, N, D] and dkpad, dvpad [D]: the sums of the
    gradients that reach pad key / value slots (zero without padding).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, D = q.shape
    zero = np.zeros(D)
    qw = _to_windows(q, grid, win, shift, None)
    kw = _to_windows(k, grid, win, shift, zero if kpad is None else kpad)
    vw = _to_windows(v, grid, win, shift, zero if vpad is None else vpad)
    dow = _to_windows(do, grid, win, shift, None)          # pad outputs are cropped: dO = 0
    dqw, dkw, dvw = attention_bwd(qw, kw, vw, dow, heads, _window_layout(B, grid, win, shift))
    real = np.zeros(_padded(grid, win), dtype=bool)
    real[:grid[0], :grid[1], :grid[2]] = True
    out = []
    for gw in (dqw, dkw, dvw):
        g = _from_windows(gw, B, grid, win, shift)
        out.append((g[:, :grid[0], :grid[1], :grid[2]].reshape(B, N, D), g[:, ~real].sum(axis=(0, 1))))
    (dq, _), (dk, dkpad), (dv, dvpad) = out
    return dq, dk, dv, dkpad, dvpad


def proxy_pool_bwd(dP: np.ndarray, grid: Grid, p: Sequence[int]) -> np.ndarray:
    """Gradient of the window average (Eq. GIIM's Averaging): every token of a
    window receives its proxy's gradient divided by P = p_t*p_h*p_w.
    dP [B, M, D] -> dx [B, N, D]."""
    dP = _f64(dP)
    B, M, D = dP.shape
    nf, nh, nw = proxy_grid(grid, p)
    P = int(np.prod(p))
    g = dP.reshape(B, nf, 1, nh, 1, nw, 1, D) / P
    g = np.broadcast_to(g, (B, nf, p[0], nh, p[1], nw, p[2], D))
    return g.reshape(B, grid[0] * grid[1] * grid[2], D).copy()


def roll3d_bwd(g: np.ndarray, shift: Sequence[int]) -> np.ndarray:
    """Gradient of the forward roll: the roll is a permutation, so its
    gradient is the inverse permutation, the roll by +s."""
    return roll3d(_f64(g), shift, inverse=True)


def linear_bwd(x: np.ndarray, w: np.ndarray, dy: np.ndarray):
    """Gradient of ptdit_oracle.linear, Y = X W^T + b (the Q/K/V/O projections
    of every attention module). x [..., d_in], w [d_out, d_in], dy [..., d_out].
    Returns dx = dY W [..., d_in], dw = dY^T X [d_out, d_in], db = sum dY [d_out]."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    x2 = x.reshape(-1, x.shape[-1])
    dy2 = dy.reshape(-1, dy.shape[-1])
    dx = (dy2 @ w).reshape(*x.shape[:-1], w.shape[1])
    return dx, dy2.T @ x2, dy2.sum(axis=0)


_NAMES = ("q", "k", "v", "o")


def _grads(d):
    """{"wq": .., "bq": .., ...} from {"q": (dW, db), ...}."""
    out = {}
    for n in _NAMES:
        out["w" + n], out["b" + n] = d[n]
    return out


def mha_bwd(xq: np.ndarray, xkv: np.ndarray, w, heads: int, dy: np.ndarray,
            allow: Optional[np.ndarray] = None):
    """Gradient of ptdit_oracle.mha(xq, xkv, w, heads, allow) for the output
    gradient dy: the output projection's linear-map gradient, the attention
    core's (attention_bwd), then the three input projections'. Returns
    (dxq, dxkv, grads) with grads = {"wq", "bq", ..., "wo", "bo"}."""
    from .ptdit_oracle import attention, linear
    q = linear(xq, w["wq"], w.get("bq"))
    k = linear(xkv, w["wk"], w.get("bk"))
    v = linear(xkv, w["wv"], w.get("bv"))
    o = attention(q, k, v, heads, allow)
    do, dwo, dbo = linear_bwd(o, w["wo"], dy)
    dq, dk, dv = attention_bwd(q, k, v, do, heads, allow)
    dxq, dwq, dbq = linear_bwd(xq, w["wq"], dq)
    dxk, dwk, dbk = linear_bwd(xkv, w["wk"], dk)
    dxv, dwv, dbv = linear_bwd(xkv, w["wv"], dv)
    return dxq, dxk + dxv, _grads({"q": (dwq, dbq), "k": (dwk, dbk), "v": (dwv, dbv), "o": (dwo, dbo)})


def window_mha_bwd(x: np.ndarray, grid: Grid, win: Sequence[int], shift: Sequence[int], w, heads: int,
                   dy: np.ndarray):
    """Gradient of the WSA (shift 0) / SWSA branch without its residual,
    Lin(window_core(Lin_q(x), Lin_k(x), Lin_v(x)); W_o, b_o), for the output
    gradient dy. Pad keys/values are the biases (reading R-bwd-pad): their
    slots' gradient sums add to d b_k, d b_v. Returns (dx, grads)."""
    from .ptdit_oracle import linear
    D = _f64(x).shape[-1]
    zero = np.zeros(D)
    bk = w.get("bk") if w.get("bk") is not None else zero
    bv = w.get("bv") if w.get("bv") is not None else zero
    q = linear(x, w["wq"], w.get("bq"))
    k = linear(x, w["wk"], w.get("bk"))
    v = linear(x, w["wv"], w.get("bv"))
    o = window_core(q, k, v, grid, win, shift, heads, bk, bv)
    do, dwo, dbo = linear_bwd(o, w["wo"], dy)
    dq, dk, dv, dkpad, dvpad = window_core_bwd(q, k, v, do, grid, win, shift, heads, bk, bv)
    dxq, dwq, dbq = linear_bwd(x, w["wq"], dq)
    dxk, dwk, dbk = linear_bwd(x, w["wk"], dk)
    dxv, dwv, dbv = linear_bwd(x, w["wv"], dv)
    return dxq + dxk + dxv, _grads({"q": (dwq, dbq), "k": (dwk, dbk + dkpad), "v": (dwv, dbv + dvpad),
                                    "o": (dwo, dbo)})


def block_bwd(x: np.ndarray, grid: Grid, p: Sequence[int], win: Sequence[int], shift: Sequence[int],
              weights, heads: int, dout: np.ndarray, pool: str = "f64"):
    """Gradient of <block(x, ...)["x3"], dout> (reading R-bwd-block).

    weights = [proxy SA, cross-attention, WSA, SWSA] as for block(); the
    forward is recomputed with the same `pool` choice. Returns {"dx": [B, N, D],
    "weights": [grads of the proxy SA, cross-attention, WSA, SWSA]}, each a
    dict of "wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo"; plus the
    intermediate gradients "dx2", "dx1", "dP2", "dP" (of x2, x1, P', P)."""
    from .ptdit_oracle import block
    f = block(x, grid, p, win, shift, weights, heads, pool=pool)
    dx3 = _f64(dout)
    dsw, g_swsa = window_mha_bwd(f["x2"], grid, win, shift, weights[3], heads, dx3)
    dx2 = dx3 + dsw                                   # x3 = x2 + SWSA(x2)
    dw, g_wsa = window_mha_bwd(f["x1"], grid, win, (0, 0, 0), weights[2], heads, dx2)
    dx1 = dx2 + dw                                    # x2 = x1 + WSA(x1)
    dxq, dP2, g_cross = mha_bwd(x, f["P2"], weights[1], heads, dx1)   # x1 = x + CS(x, P')
    dPq, dPkv, g_sa = mha_bwd(f["P"], f["P"], weights[0], heads, dP2)  # P' = P + SA(P)
    dP = dP2 + dPq + dPkv
    dx = dx1 + dxq + proxy_pool_bwd(dP, grid, p)      # P = Averaging(x)
    return {"dx": dx, "weights": [g_sa, g_cross, g_wsa, g_swsa], "dx2": dx2, "dx1": dx1, "dP2": dP2, "dP": dP}
