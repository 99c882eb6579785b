"""Float64 NumPy oracle of the PT-DiT attention core (GIIM + TCM).

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the GPU path.

Source of every step: the Qihoo-T2X reading note (page "Qihoo-T2X —
Proxy-Tokenized DiT for Text-to-Any-Task"), section 3 "Method":
  * Eq. GIIM: z_s = CS(z_s, SA(Averaging(z_s))), with z_s reshaped to f x h x w
    and one proxy per p_t x p_h x p_w window (window average);
  * Eq. TCM: z_hat = WSA(z_s) + z_s ; z_w = SWSA(z_hat) + z_hat;
  * the code-correspondence section, excerpt 2 (PT-Block forward), for the
    order GIIM -> TCM and the residual placement (proxy SA adds its input,
    the cross-attention output goes through one more linear and is added to
    the token stream, window attention adds its input, shifted-window
    attention is a cyclic shift, window attention and the inverse shift);
  * the "complexity" paragraph of section 3 for the attention-cost formula.

Readings where the pages are silent (each named below; the tests refer to them by name):
  R-order   tokens are row-major over (f, h, w); proxies row-major over the
            window grid (Figure 2 notes: row-major flattening).
  R-pool32  the window average's kernel precision: float32 sums taken along
            the w axis in index order, those row sums added over h in index
            order, those over t in index order, then one IEEE float32
            division by P = p_t*p_h*p_w; a bf16 output rounds to nearest even.
  R-norm    the norms in front of each attention are identity (never given).
  R-out     to_out followed by linear_1_visual is one linear map: one output
            projection (W_o, b_o) per attention.
  R-kv      cross-attention keys/values come from the attended proxies P'.
  R-scale   scale 1/sqrt(d_h); head h owns channels [h*d_h, (h+1)*d_h); no
            positional term inside the core.
  R-pad     TCM zero-pads its own input grid at the high end of every axis to a
            multiple of the window; pad tokens take part as keys/values; pad
            outputs are cropped. Padding comes before the shift.
  R-shift   SWSA rolls the padded grid by -s, z[k] = y[(k + s) mod L];
            windows start at the origin of the rolled grid; the inverse roll
            is by +s.
  R-mask    boundary mask in rolled coordinates: per axis of length L with
            window w and shift s the region of coordinate k is 0 if k < L-w,
            1 if L-w <= k < L-s, 2 otherwise; a query sees a key only if their
            regions agree on every axis; excluded pairs get weight exactly 0.
  R-select  the proxy-extraction ablation's Top-Left and Random proxies (and
            get_proxy_token's mode "first", code-correspondence excerpt 1)
            take one token of the window as its proxy: the token at the
            window-local offset o = (dt*p_h + di)*p_w + dj (row-major inside
            the window, as R-order), o = 0 for Top-Left, a drawn offset per
            window for Random; offsets are taken modulo P.
  R-text    the text cross-attention after TCM (section 3: PT-Block = GIIM +
            TCM + text cross-attn + MLP; Figure 3 data flow) is MHA with the
            tokens as queries and the caption embeddings (already projected to
            D, outside the block like the patch embedding) as keys/values,
            plus the residual: the same map as the proxy cross-attention.
  R-mlp     the MLP is the DiT/PixArt feed-forward: Lin(GELU(Lin(x; W1, b1));
            W2, b2) with hidden width 4D and the tanh form of GELU, plus the
            residual. The pages name the MLP and nothing about its shape.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "precision", "linear", "attention", "mha", "proxy_grid", "proxy_pool", "proxy_pool_f32", "proxy_select",
    "round_bf16_rne", "proxy_sa", "proxy_xattn", "pad_grid", "partition",
    "unpartition", "roll3d", "region_labels", "window_sa", "shift_window_sa",
    "block", "count_core_macs", "count_projection_macs", "gelu_tanh", "mlp", "text_xattn",
]

Grid = Tuple[int, int, int]
Weights = Dict[str, np.ndarray]


# Working precision of every step: float64, except inside `precision()`.
_DT = np.float64


class precision:
    """Context manager that runs the same arithmetic in another NumPy float
    type, e.g. ``with precision(np.float32): block(...)``. Only the CPU
    baseline uses it (the fp32 NumPy oracle the target statement names); every
    pin and parity test uses the float64 default."""

    def __init__(self, dtype):
        self.dtype = np.dtype(dtype).type
        self.saved = None

    def __enter__(self):
        global _DT
        self.saved, _DT = _DT, self.dtype
        return self

    def __exit__(self, *exc):
        global _DT
        _DT = self.saved
        return False


def _f64(a) -> np.ndarray:
    """The working precision (float64 unless inside `precision`)."""
    return np.asarray(a, dtype=_DT)


# ----------------------------------------------------------------------------
# Linear maps and multi-head attention
# ----------------------------------------------------------------------------

def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """Lin(X; W, b) = X W^T + b over the last axis (nn.Linear convention).

    The Q/K/V/O projections of every attention module named in the code
    correspondence table (proxy_attn1, pvisual_attn2, attn1) are such maps.
    """
    x = _f64(x)
    lead = x.shape[:-1]
    y = x.reshape(-1, x.shape[-1]) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)
    return y.reshape(*lead, y.shape[-1])


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, heads: int,
              allow: Optional[np.ndarray] = None) -> np.ndarray:
    """Scaled dot-product attention, head by head (reading R-scale).

    q: [..., Lq, D]; k, v: [..., Lk, D]; allow: broadcastable to [..., Lq, Lk]
    (True = the query may see the key). For head h: S = Q_h K_h^T / sqrt(d_h),
    excluded pairs are removed (weight exactly 0), A = softmax over keys,
    O_h = A V_h. Returns concat_h O_h, [..., Lq, D].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    D = q.shape[-1]
    dh = D // heads
    out = np.empty(q.shape[:-1] + (D,), dtype=_DT)
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        s = (q[..., sl] @ np.swapaxes(k[..., sl], -1, -2)) / float(np.sqrt(dh))
        if allow is not None:
            s = np.where(allow, s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=-1, keepdims=True)
        out[..., sl] = a @ v[..., sl]
    return out


def mha(xq: np.ndarray, xkv: np.ndarray, w: Weights, heads: int,
        allow: Optional[np.ndarray] = None) -> np.ndarray:
    """Multi-head attention with its four projections (readings R-out, R-scale).

    Q = Lin(xq; Wq, bq), K = Lin(xkv; Wk, bk), V = Lin(xkv; Wv, bv);
    output Lin(attention(Q, K, V); Wo, bo).
    """
    q = linear(xq, w["wq"], w.get("bq"))
    k = linear(xkv, w["wk"], w.get("bk"))
    v = linear(xkv, w["wv"], w.get("bv"))
    o = attention(q, k, v, heads, allow)
    return linear(o, w["wo"], w.get("bo"))


# ----------------------------------------------------------------------------
# GIIM: window-average proxies, proxy self-attention, cross-attention
# ----------------------------------------------------------------------------

def proxy_grid(grid: Grid, p: Sequence[int]) -> Grid:
    F, H, W = grid
    if F % p[0] or H % p[1] or W % p[2]:
        raise ValueError(f"proxy window {tuple(p)} does not divide grid {grid}")
    return (F // p[0], H // p[1], W // p[2])


def proxy_pool(x: np.ndarray, grid: Grid, p: Sequence[int]) -> np.ndarray:
    """Averaging(z_s) of Eq. GIIM: one proxy per p_t x p_h x p_w window.

    x: [B, N, D] with tokens row-major over (f, h, w). Proxy (T, I, J) is the
    float64 mean of the tokens (T*p_t + dt, I*p_h + di, J*p_w + dj); proxies
    are row-major over (T, I, J) (reading R-order). Returns [B, M, D].
    """
    x = _f64(x)
    B, N, D = x.shape
    FT, HI, WJ = proxy_grid(grid, p)
    xg = x.reshape(B, FT, p[0], HI, p[1], WJ, p[2], D)
    return xg.mean(axis=(2, 4, 6)).reshape(B, FT * HI * WJ, D)


def proxy_select(x: np.ndarray, grid: Grid, p: Sequence[int],
                 offsets: Optional[np.ndarray] = None) -> np.ndarray:
    """One token per window as its proxy (reading R-select): the alternative
    to Averaging in the proxy-extraction ablation (section 3, ablation notes).

    x: [B, N, D]; offsets: [B, M] window-local offsets (taken modulo P) or
    None for every window's top-left token. Returns [B, M, D] (float64 values
    of the selected tokens, no arithmetic).
    """
    x = _f64(x)
    B, N, D = x.shape
    FT, HI, WJ = proxy_grid(grid, p)
    P = p[0] * p[1] * p[2]
    xg = x.reshape(B, FT, p[0], HI, p[1], WJ, p[2], D)
    # [B, M, P, D]: the window's tokens in row-major (dt, di, dj) order
    win = xg.transpose(0, 1, 3, 5, 2, 4, 6, 7).reshape(B, FT * HI * WJ, P, D)
    if offsets is None:
        return win[:, :, 0, :].copy()
    o = np.mod(np.asarray(offsets, dtype=np.int64), P).reshape(B, FT * HI * WJ)
    return np.take_along_axis(win, o[:, :, None, None], axis=2)[:, :, 0, :]


def proxy_pool_f32(x: np.ndarray, grid: Grid, p: Sequence[int]) -> np.ndarray:
    """The same window average in the kernel's precision (reading R-pool32).

    Sums are float32: for every (dt, di) the row sum over dj is taken in index
    order starting from 0; the row sums are added over di in index order; the
    plane sums over dt in index order; then one IEEE float32 division by P.
    NumPy float32 addition and division round correctly, elementwise.
    Returns float32 [B, M, D].
    """
    x32 = np.asarray(x, dtype=np.float32)
    B, N, D = x32.shape
    FT, HI, WJ = proxy_grid(grid, p)
    xg = x32.reshape(B, FT, p[0], HI, p[1], WJ, p[2], D)
    total = np.zeros((B, FT, HI, WJ, D), dtype=np.float32)
    for dt in range(p[0]):
        plane = np.zeros_like(total)
        for di in range(p[1]):
            row = np.zeros_like(total)
            for dj in range(p[2]):
                row = row + xg[:, :, dt, :, di, :, dj, :]
            plane = plane + row
        total = total + plane
    mean = total / np.float32(p[0] * p[1] * p[2])
    return mean.reshape(B, FT * HI * WJ, D)


def round_bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest, ties to even; returns float32.

    bf16 keeps the top 16 bits of the float32 pattern. Adding 0x7FFF plus the
    lowest kept bit before truncating rounds to nearest with ties to even.
    NaN inputs stay NaN (quietened).
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = r.astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, (f.view(np.uint32) | 0x00400000) & 0xFFFF0000, r).astype(np.uint32)
    return r.view(np.float32)


def proxy_sa(P: np.ndarray, w: Weights, heads: int, residual: bool = True) -> np.ndarray:
    """Proxy self-attention of GIIM: P' = P + MHA(P, P) (excerpt 2 adds the
    input back; reading R-norm for the proxy norm). P: [B, M, D]."""
    y = mha(P, P, w, heads)
    return _f64(P) + y if residual else y


def proxy_xattn(x: np.ndarray, P2: np.ndarray, w: Weights, heads: int,
                residual: bool = True) -> np.ndarray:
    """CS(z_s, P') of Eq. GIIM: every latent token is a query, the attended
    proxies P' are keys and values (reading R-kv); the output projection plays
    linear_1_visual's role (reading R-out) and is added to the token stream."""
    y = mha(x, P2, w, heads)
    return _f64(x) + y if residual else y


def text_xattn(x: np.ndarray, text: np.ndarray, w: Weights, heads: int,
               residual: bool = True) -> np.ndarray:
    """Text cross-attention of the PT-Block (reading R-text): tokens are
    queries, caption embeddings [B, L, D] are keys and values."""
    y = mha(x, text, w, heads)
    return _f64(x) + y if residual else y


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU in its tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
    (Hendrycks & Gimpel, the approximation DiT-style MLPs use)."""
    x = _f64(x)
    return 0.5 * x * (1.0 + np.tanh(float(np.sqrt(2.0 / np.pi)) * (x + 0.044715 * x ** 3)))


def mlp(x: np.ndarray, w: Weights, residual: bool = True) -> np.ndarray:
    """The PT-Block's MLP (reading R-mlp): Lin(GELU(Lin(x; W1, b1)); W2, b2)
    (+ x). w = {"w1": [H, D], "b1": [H], "w2": [D, H], "b2": [D]}."""
    y = linear(gelu_tanh(linear(x, w["w1"], w.get("b1"))), w["w2"], w.get("b2"))
    return _f64(x) + y if residual else y


# ----------------------------------------------------------------------------
# TCM: window attention and shifted-window attention
# ----------------------------------------------------------------------------

def _padded(grid: Grid, win: Sequence[int]) -> Grid:
    return tuple(-(-g // w) * w for g, w in zip(grid, win))


def pad_grid(x: np.ndarray, grid: Grid, win: Sequence[int]) -> np.ndarray:
    """[B, N, D] -> [B, F', H', W', D], zero tokens appended at the high end of
    every axis up to a multiple of the window (reading R-pad)."""
    x = _f64(x)
    B, N, D = x.shape
    Fp, Hp, Wp = _padded(grid, win)
    out = np.zeros((B, Fp, Hp, Wp, D), dtype=_DT)
    out[:, :grid[0], :grid[1], :grid[2]] = x.reshape(B, *grid, D)
    return out


def partition(xg: np.ndarray, win: Sequence[int]) -> np.ndarray:
    """[B, F', H', W', C...] -> [B, nT, nH, nW, w_t*w_h*w_w, C...]: windows of
    w_t x w_h x w_w starting at the origin, tokens row-major inside a window."""
    B, Fp, Hp, Wp = xg.shape[:4]
    rest = xg.shape[4:]
    wt, wh, ww = win
    y = xg.reshape(B, Fp // wt, wt, Hp // wh, wh, Wp // ww, ww, *rest)
    y = np.moveaxis(y, (2, 4, 6), (4, 5, 6))
    return y.reshape(B, Fp // wt, Hp // wh, Wp // ww, wt * wh * ww, *rest)


def unpartition(xw: np.ndarray, win: Sequence[int]) -> np.ndarray:
    """Inverse of partition."""
    B, nT, nH, nW, L = xw.shape[:5]
    rest = xw.shape[5:]
    wt, wh, ww = win
    y = xw.reshape(B, nT, nH, nW, wt, wh, ww, *rest)
    y = np.moveaxis(y, (4, 5, 6), (2, 4, 6))
    return y.reshape(B, nT * wt, nH * wh, nW * ww, *rest)


def roll3d(xg: np.ndarray, shift: Sequence[int], inverse: bool = False) -> np.ndarray:
    """Cyclic roll of a grid [B, F, H, W, ...] (reading R-shift).

    Forward: z[t, i, j] = y[(t + s_t) mod F, (i + s_h) mod H, (j + s_w) mod W].
    Inverse: z[t, i, j] = y[(t - s_t) mod F, ...], so inverse(forward(y)) = y.
    Written as an explicit index gather along each axis.
    """
    sgn = -1 if inverse else 1
    out = xg
    for axis, s in zip((1, 2, 3), shift):
        L = out.shape[axis]
        idx = (np.arange(L) + sgn * s) % L
        out = np.take(out, idx, axis=axis)
    return out


def region_labels(padded: Grid, win: Sequence[int], shift: Sequence[int]) -> np.ndarray:
    """Boundary-mask labels on the rolled padded grid (reading R-mask).

    Per axis of length L: region 0 if k < L - w, 1 if L - w <= k < L - s,
    2 otherwise; the token's label combines the three axes' regions.
    Returns int [F', H', W'].
    """
    labs = []
    for L, w, s in zip(padded, win, shift):
        k = np.arange(L)
        r = np.where(k < L - w, 0, np.where(k < L - s, 1, 2))
        labs.append(r)
    return (labs[0][:, None, None] * 9 + labs[1][None, :, None] * 3 + labs[2][None, None, :])


def window_sa(x: np.ndarray, grid: Grid, win: Sequence[int], w: Weights, heads: int,
              residual: bool = True) -> np.ndarray:
    """WSA of Eq. TCM: attention inside each window of the zero-padded grid,
    cropped back to the real tokens; z_hat = WSA(z) + z with residual."""
    x = _f64(x)
    B, N, D = x.shape
    xp = pad_grid(x, grid, win)
    xw = partition(xp, win)                       # [B, nT, nH, nW, L, D]
    lead = xw.shape[:4]
    xw = xw.reshape(-1, xw.shape[4], D)
    ow = mha(xw, xw, w, heads).reshape(*lead, -1, D)
    y = unpartition(ow, win)[:, :grid[0], :grid[1], :grid[2]].reshape(B, N, D)
    return x + y if residual else y


def shift_window_sa(x: np.ndarray, grid: Grid, win: Sequence[int], shift: Sequence[int],
                    w: Weights, heads: int, residual: bool = True) -> np.ndarray:
    """SWSA of Eq. TCM: pad, roll by -s, window attention under the boundary
    mask, roll back by +s, crop; z_w = SWSA(z_hat) + z_hat with residual."""
    x = _f64(x)
    B, N, D = x.shape
    xp = pad_grid(x, grid, win)
    padded = xp.shape[1:4]
    z = roll3d(xp, shift)
    zw = partition(z, win)
    lead = zw.shape[:4]
    L = zw.shape[4]
    zw = zw.reshape(-1, L, D)
    lab = partition(region_labels(padded, win, shift)[None, ..., None], win)
    lab = np.broadcast_to(lab.reshape(-1, L), (B,) + lab.reshape(-1, L).shape).reshape(-1, L)
    allow = lab[:, :, None] == lab[:, None, :]
    ow = mha(zw, zw, w, heads, allow).reshape(*lead, L, D)
    y = roll3d(unpartition(ow, win), shift, inverse=True)
    y = y[:, :grid[0], :grid[1], :grid[2]].reshape(B, N, D)
    return x + y if residual else y


# ----------------------------------------------------------------------------
# The block's attention core and its cost
# ----------------------------------------------------------------------------

def block(x: np.ndarray, grid: Grid, p: Sequence[int], win: Sequence[int],
          shift: Sequence[int], weights: Sequence[Weights], heads: int,
          pool: str = "f64", offsets: Optional[np.ndarray] = None,
          text: Optional[np.ndarray] = None, w_text: Optional[Weights] = None,
          w_mlp: Optional[Weights] = None) -> Dict[str, np.ndarray]:
    """GIIM then TCM, in the order of excerpt 2 (PT-Block forward).

    weights = [proxy SA, cross-attention, WSA, SWSA]. pool="f64" uses the
    float64 window mean; pool="bf16" uses the kernel-precision mean rounded to
    bf16 (what a bf16 proxy tensor holds); pool="select" takes one token per
    window (reading R-select; offsets None: top-left). Returns every
    intermediate.
    """
    if pool == "select":
        P = proxy_select(x, grid, p, offsets)
    elif pool == "f64":
        P = proxy_pool(x, grid, p)
    elif pool == "bf16":
        P = _f64(round_bf16_rne(proxy_pool_f32(x, grid, p)))
    elif pool == "f32":
        P = _f64(proxy_pool_f32(x, grid, p))
    else:
        raise ValueError(pool)
    P2 = proxy_sa(P, weights[0], heads)
    x1 = proxy_xattn(x, P2, weights[1], heads)
    x2 = window_sa(x1, grid, win, weights[2], heads)
    x3 = shift_window_sa(x2, grid, win, shift, weights[3], heads)
    out = {"P": P, "P2": P2, "x1": x1, "x2": x2, "x3": x3}
    # the rest of the PT-Block (readings R-text, R-mlp), when given
    if text is not None:
        out["x4"] = text_xattn(x3, text, w_text, heads)
        out["x5"] = mlp(out["x4"], w_mlp)
    return out


def count_core_macs(grid: Grid, p: Sequence[int], win: Sequence[int], D: int,
                    B: int = 1, real_queries: bool = False) -> Dict[str, int]:
    """Multiply-accumulates of the attention cores (Q K^T plus A V), counted
    over the same partitions the oracle computes on (dense windows, mask not
    skipped), for comparison with the complexity paragraph's formula.

    With real_queries=True only queries that are real tokens are counted
    (keys still include pad tokens).
    """
    M = int(np.prod(proxy_grid(grid, p)))
    # partition an index grid exactly as window_sa / shift_window_sa do
    padded = _padded(grid, win)
    real = np.zeros(padded, dtype=bool)
    real[:grid[0], :grid[1], :grid[2]] = True
    rw = partition(real[None, ..., None], win).reshape(-1, int(np.prod(win)))
    nq = rw.sum(axis=1) if real_queries else np.full(rw.shape[0], rw.shape[1])
    win_macs = int(np.sum(2 * nq.astype(np.int64) * rw.shape[1] * D)) * B
    return {
        "proxy_sa": B * 2 * M * M * D,
        "xattn": B * 2 * int(np.prod(grid)) * M * D,
        "wsa": win_macs,
        "swsa": win_macs,
    }


def count_projection_macs(grid: Grid, p: Sequence[int], win: Sequence[int], D: int,
                          B: int = 1, padded_rows: bool = False) -> Dict[str, int]:
    """Multiply-accumulates of the Q/K/V/O projections of the four attentions.

    With padded_rows=False, projections of pad tokens are not counted (they
    reduce to the bias); with True they are.
    """
    N = int(np.prod(grid))
    M = int(np.prod(proxy_grid(grid, p)))
    rows = int(np.prod(_padded(grid, win))) if padded_rows else N
    DD = D * D
    return {
        "proxy_sa": B * (3 * M + M) * DD,
        "xattn": B * (N + 2 * M + N) * DD,
        "wsa": B * (3 * rows + N) * DD,
        "swsa": B * (3 * rows + N) * DD,
    }
