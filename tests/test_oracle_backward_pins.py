"""Pins of the float64 backward oracle against things other than itself.

CPU only. The backward oracle (oracle/ptdit_backward.py) is checked against:
  * central finite differences of the (separately pinned) forward oracle, one
    directional derivative per argument, so a wrong sign, a dropped term or a
    transposed operand in any one gradient fails;
  * torch's autograd through scaled_dot_product_attention and linear in
    float64 (library routines with their own backward);
  * closed forms: uniform attention (Q = 0) and the window average's adjoint;
  * adjoint identities <f(x), y> = <x, f^T(y)> for the pooling and the roll,
    and numpy.roll for the roll's inverse.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _allow(g, Lq, Lk, lead=()):
    a = g.random(lead + (Lq, Lk)) < 0.6
    a[..., 0] |= ~a.any(axis=-1)  # every query sees at least one key
    return a


def _fd(f, args, i, d, eps=1e-5):
    """Central difference of scalar f along direction d of argument i."""
    p = list(args)
    m = list(args)
    p[i] = args[i] + eps * d
    m[i] = args[i] - eps * d
    return (f(*p) - f(*m)) / (2 * eps)


@pytest.mark.parametrize("masked", [False, True])
def test_attention_bwd_matches_finite_differences(masked):
    g = _rng(11 + masked)
    Lq, Lk, D, heads = 5, 7, 8, 2
    q, k, v, do = (g.standard_normal((2, L, D)) for L in (Lq, Lk, Lk, Lq))
    allow = _allow(g, Lq, Lk, (2,)) if masked else None
    loss = lambda q_, k_, v_: float((O.attention(q_, k_, v_, heads, allow) * do).sum())
    grads = O.attention_bwd(q, k, v, do, heads, allow)
    for i, gr in enumerate(grads):
        d = g.standard_normal(gr.shape)
        fd = _fd(loss, (q, k, v), i, d)
        assert abs(fd - (gr * d).sum()) <= 1e-7 * max(1.0, abs(fd)), (i, fd, (gr * d).sum())


def test_attention_bwd_matches_torch_autograd():
    g = _rng(21)
    B, heads, Lq, Lk, dh = 2, 3, 6, 9, 4
    D = heads * dh
    q, k, v, do = (g.standard_normal((B, L, D)) for L in (Lq, Lk, Lk, Lq))
    allow = _allow(g, Lq, Lk, (B,))
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    split = lambda t, L: t.reshape(B, L, heads, dh).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        split(tq, Lq), split(tk, Lk), split(tv, Lk), attn_mask=torch.tensor(allow)[:, None])
    o = o.transpose(1, 2).reshape(B, Lq, D)
    o.backward(torch.tensor(do))
    dq, dk, dv = O.attention_bwd(q, k, v, do, heads, allow)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_bwd_uniform_closed_form():
    # Q = 0: every allowed weight is 1/n. Then dV_j = mean_i dO_i, dK = 0, and
    # dQ_i = scale/n * (sum_j a_ij k_j - mean_j(a_ij) sum_j k_j), a_ij = dO_i . v_j.
    g = _rng(31)
    L, D = 6, 5
    q = np.zeros((L, D))
    k, v, do = (g.standard_normal((L, D)) for _ in range(3))
    dq, dk, dv = O.attention_bwd(q, k, v, do, 1)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=0), (L, D)), atol=1e-14)
    np.testing.assert_allclose(dk, 0, atol=1e-14)
    a = do @ v.T
    ref = (a @ k - a.mean(axis=1, keepdims=True) * k.sum(axis=0)) / L / np.sqrt(D)
    np.testing.assert_allclose(dq, ref, atol=1e-13)


CORE_CASES = [
    # (B, grid, win, shift): padding on every axis and a shift; no padding
    # without a shift; a video grid with a temporal window
    (1, (1, 6, 7), (1, 4, 4), (0, 2, 2)),
    (2, (1, 4, 8), (1, 4, 4), (0, 0, 0)),
    (1, (3, 4, 5), (2, 2, 4), (1, 1, 2)),
]


@pytest.mark.parametrize("case", CORE_CASES)
def test_window_core_is_the_forward_core(case):
    B, grid, win, shift = case
    g = _rng(41)
    D, heads = 8, 2
    x = g.standard_normal((B, int(np.prod(grid)), D))
    w = {n: g.standard_normal((D, D)) * 0.4 for n in ("wq", "wk", "wv", "wo")}
    w.update({n: g.standard_normal(D) * 0.4 for n in ("bq", "bk", "bv", "bo")})
    q, k, v = (O.linear(x, w["w" + c], w["b" + c]) for c in "qkv")
    o = O.window_core(q, k, v, grid, win, shift, heads, w["bk"], w["bv"])
    ref = (O.shift_window_sa(x, grid, win, shift, w, heads, residual=False) if any(shift)
           else O.window_sa(x, grid, win, w, heads, residual=False))
    np.testing.assert_allclose(O.linear(o, w["wo"], w["bo"]), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("case", CORE_CASES)
def test_window_core_bwd_matches_finite_differences(case):
    B, grid, win, shift = case
    g = _rng(51)
    D, heads = 8, 2
    N = int(np.prod(grid))
    q, k, v, do = (g.standard_normal((B, N, D)) for _ in range(4))
    kp, vp = g.standard_normal(D), g.standard_normal(D)
    loss = lambda q_, k_, v_, kp_, vp_: float((O.window_core(q_, k_, v_, grid, win, shift, heads, kp_, vp_)
                                               * do).sum())
    grads = O.window_core_bwd(q, k, v, do, grid, win, shift, heads, kp, vp)
    padded = any(-(-s // w) * w != s for s, w in zip(grid, win))
    for i, gr in enumerate(grads):
        d = g.standard_normal(gr.shape)
        fd = _fd(loss, (q, k, v, kp, vp), i, d)
        assert abs(fd - (gr * d).sum()) <= 1e-7 * max(1.0, abs(fd)), (i, fd, (gr * d).sum())
        if i >= 3 and not padded:
            np.testing.assert_array_equal(gr, 0)


def test_pool_bwd_is_the_adjoint_of_the_window_average():
    g = _rng(61)
    grid, p, D = (2, 4, 6), (2, 2, 3), 5
    x = g.standard_normal((2, int(np.prod(grid)), D))
    gp = g.standard_normal((2, 4, D))
    lhs = (O.proxy_pool(x, grid, p) * gp).sum()
    rhs = (x * O.proxy_pool_bwd(gp, grid, p)).sum()
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # one-hot proxy gradient: exactly 1/P on its window's 12 tokens, 0 elsewhere
    one = np.zeros((1, 4, 1))
    one[0, 3, 0] = 1.0
    dx = O.proxy_pool_bwd(one, grid, p).reshape(*grid)
    assert np.count_nonzero(dx) == 12 and np.all(dx[1:, 2:, 3:] == 1 / 12)


def test_roll_bwd_is_the_adjoint_and_numpy_roll():
    g = _rng(71)
    shift = (1, 2, 3)
    x = g.standard_normal((1, 3, 5, 7, 2))
    y = g.standard_normal((1, 3, 5, 7, 2))
    lhs = (O.roll3d(x, shift) * y).sum()
    rhs = (x * O.roll3d_bwd(y, shift)).sum()
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    np.testing.assert_array_equal(O.roll3d_bwd(y, shift), np.roll(y, shift, axis=(1, 2, 3)))


def test_linear_bwd_matches_torch_autograd_and_finite_differences():
    g = _rng(81)
    x, w, dy = g.standard_normal((2, 5, 6)), g.standard_normal((4, 6)), g.standard_normal((2, 5, 4))
    b = g.standard_normal(4)
    tx, tw, tb = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, w, b))
    torch.nn.functional.linear(tx, tw, tb).backward(torch.tensor(dy))
    dx, dw, db = O.linear_bwd(x, w, dy)
    for mine, ref in ((dx, tx.grad), (dw, tw.grad), (db, tb.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-12, atol=1e-12)
    loss = lambda x_, w_, b_: float((O.linear(x_, w_, b_) * dy).sum())
    for i, gr in enumerate((dx, dw, db)):
        d = g.standard_normal(gr.shape)
        fd = _fd(loss, (x, w, b), i, d)
        assert abs(fd - (gr * d).sum()) <= 1e-7 * max(1.0, abs(fd))
