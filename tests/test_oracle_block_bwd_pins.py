"""Pins of the oracle's block backward (oracle.block_bwd, reading R-bwd-block):
the gradient of <x3, dout> with respect to the block input and all 32 weight
and bias tensors of the four attentions, chained from the pinned per-op
gradients. Two independent checks:
  * central finite differences of the float64 forward oracle (oracle.block),
    one random direction per argument;
  * torch autograd (float64, CPU) through a separate restatement of the
    block forward built from torch library routines (avg_pool3d,
    scaled_dot_product_attention with boolean masks, torch.roll, F.pad).
Grids cover TCM padding on every axis, a shift that differs from the pad,
3D windows, batch 2, and p_t > 1 (temporal proxy windows).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import oracle as O
from synth_inputs import make_all_weights, make_x, tiny

NAMES = ("wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo")

CASES = {
    # grid (B, F, H, W), D, heads, p, win, shift
    "video_pad_shift": ((1, 2, 5, 6), 16, 2, (1, 5, 3), (2, 4, 4), (1, 2, 2)),
    "img_pad_noniso": ((1, 1, 10, 12), 16, 2, (1, 5, 4), (1, 4, 4), (0, 1, 2)),
    "batch2_temporal_proxy": ((2, 4, 4, 4), 8, 2, (2, 2, 2), (2, 2, 4), (1, 1, 0)),
}


def _case(name):
    (B, F, H, W), D, heads, p, win, shift = CASES[name]
    wl = tiny(name, B=B, F=F, H=H, W=W, D=D, heads=heads, p=p, win=win, shift=shift, index=70 + len(name))
    x = make_x(wl).astype(np.float64)
    ws = [{k: v.astype(np.float64) * 10.0 for k, v in w.items()} for w in make_all_weights(wl)]  # O(1) scores
    g = np.random.default_rng(5 + len(name))
    dout = g.standard_normal((B, wl.N, D))
    return wl, x, ws, dout


def _loss(wl, x, ws, dout):
    return float(np.sum(O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads)["x3"] * dout))


@pytest.mark.parametrize("name", list(CASES))
def test_block_bwd_matches_finite_differences(name):
    wl, x, ws, dout = _case(name)
    r = O.block_bwd(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads, dout)
    g = np.random.default_rng(11)
    eps = 1e-5

    def check(analytic, perturb):
        u = g.standard_normal(analytic.shape)
        lp, lm = perturb(u * eps), perturb(-u * eps)
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(analytic * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)

    check(r["dx"], lambda d: _loss(wl, x + d, ws, dout))
    for a in range(4):
        for n in NAMES:
            def pert(d, a=a, n=n):
                w2 = [dict(w) for w in ws]
                w2[a][n] = ws[a][n] + d
                return _loss(wl, x, w2, dout)
            check(r["weights"][a][n], pert)


def _torch_block(x, grid, p, win, shift, ws, heads):
    """The block forward restated with torch library routines (float64)."""
    B, N, D = x.shape
    F, H, W = grid
    dh = D // heads

    def mha(xq, xkv, w, mask=None):
        q, k, v = (TF.linear(xq, w["wq"], w["bq"]), TF.linear(xkv, w["wk"], w["bk"]),
                   TF.linear(xkv, w["wv"], w["bv"]))
        sp = lambda t: t.reshape(*t.shape[:-1], heads, dh).transpose(-2, -3)
        o = TF.scaled_dot_product_attention(sp(q), sp(k), sp(v), attn_mask=mask)
        return TF.linear(o.transpose(-2, -3).reshape(*xq.shape[:-1], D), w["wo"], w["bo"])

    def windows(y, w, s):
        Fp, Hp, Wp = (-(-F // win[0]) * win[0], -(-H // win[1]) * win[1], -(-W // win[2]) * win[2])
        yg = y.reshape(B, F, H, W, D)
        yg = TF.pad(yg, (0, 0, 0, Wp - W, 0, Hp - H, 0, Fp - F))        # zero tokens at the high ends
        if any(s):
            yg = torch.roll(yg, shifts=(-s[0], -s[1], -s[2]), dims=(1, 2, 3))
        nf, nh, nw = Fp // win[0], Hp // win[1], Wp // win[2]
        L = win[0] * win[1] * win[2]
        t = yg.reshape(B, nf, win[0], nh, win[1], nw, win[2], D).permute(0, 1, 3, 5, 2, 4, 6, 7).reshape(-1, L, D)
        mask = None
        if any(s):
            def reg(Lp, ww, ss):   # rolled coordinate -> boundary region on one axis
                k = torch.arange(Lp)
                return (k >= Lp - ww).long() + (k >= Lp - ss).long()
            lab = (reg(Fp, win[0], s[0])[:, None, None] * 9 + reg(Hp, win[1], s[1])[None, :, None] * 3
                   + reg(Wp, win[2], s[2])[None, None, :])
            lab = lab.reshape(nf, win[0], nh, win[1], nw, win[2]).permute(0, 2, 4, 1, 3, 5).reshape(-1, L)
            mask = (lab[:, :, None] == lab[:, None, :]).repeat(B, 1, 1)[:, None]
        o = mha(t, t, w, mask)
        og = o.reshape(B, nf, nh, nw, win[0], win[1], win[2], D).permute(0, 1, 4, 2, 5, 3, 6, 7)
        og = og.reshape(B, Fp, Hp, Wp, D)
        if any(s):
            og = torch.roll(og, shifts=tuple(s), dims=(1, 2, 3))
        return og[:, :F, :H, :W].reshape(B, N, D)

    xg = x.reshape(B, F, H, W, D).permute(0, 4, 1, 2, 3)
    P = TF.avg_pool3d(xg, kernel_size=tuple(p), stride=tuple(p)).permute(0, 2, 3, 4, 1).reshape(B, -1, D)
    P2 = P + mha(P, P, ws[0])
    x1 = x + mha(x, P2, ws[1])
    x2 = x1 + windows(x1, ws[2], (0, 0, 0))
    return x2 + windows(x2, ws[3], shift)


@pytest.mark.parametrize("name", list(CASES))
def test_block_bwd_matches_torch_autograd(name):
    wl, x, ws, dout = _case(name)
    r = O.block_bwd(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads, dout)
    xt = torch.tensor(x, requires_grad=True)
    wt = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in ws]
    y = _torch_block(xt, wl.grid, wl.p, wl.win, wl.shift, wt, wl.heads)
    ref_fwd = O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads)["x3"]
    np.testing.assert_allclose(y.detach().numpy(), ref_fwd, rtol=1e-10, atol=1e-10)
    (y * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(r["dx"], xt.grad.numpy(), rtol=1e-9, atol=1e-9)
    for a in range(4):
        for n in NAMES:
            np.testing.assert_allclose(r["weights"][a][n], wt[a][n].grad.numpy(), rtol=1e-9, atol=1e-9,
                                       err_msg=f"attention {a} {n}")


def test_block_bwd_planted_mistakes_fail():
    """The torch pin catches plausible slips in the chain: the cross-attention
    gradient not fed back through P' into the window average, and the WSA
    residual's pass-through dropped."""
    wl, x, ws, dout = _case("img_pad_noniso")
    xt = torch.tensor(x, requires_grad=True)
    wt = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in ws]
    (_torch_block(xt, wl.grid, wl.p, wl.win, wl.shift, wt, wl.heads) * torch.tensor(dout)).sum().backward()
    ref = xt.grad.numpy()
    f = O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads)
    dsw, _ = O.window_mha_bwd(f["x2"], wl.grid, wl.win, wl.shift, ws[3], wl.heads, dout)
    dx2 = dout + dsw
    dw, _ = O.window_mha_bwd(f["x1"], wl.grid, wl.win, (0, 0, 0), ws[2], wl.heads, dx2)
    dxq, dP2, _ = O.mha_bwd(x, f["P2"], ws[1], wl.heads, dx2 + dw)
    no_pool = dx2 + dw + dxq                                   # P' path dropped
    no_res = dw + dxq + O.proxy_pool_bwd(dP2, wl.grid, wl.p)   # residual of WSA dropped (and P path partly)
    for bad in (no_pool, no_res):
        assert np.abs(bad - ref).max() > 1e-3
