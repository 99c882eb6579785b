"""Pins of the float64 oracle against things other than itself.

Every test here runs on the CPU (no GPU marker). Each pin is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong roll direction or mask region) fails at least one:
  * library routines: torch's scaled_dot_product_attention / linear (fp64),
    numpy.roll, torch's bf16 cast;
  * closed forms: one-proxy GIIM, uniform attention (W_k = 0), one-token
    windows, window-mean of V;
  * exact rational checks of the float32 window average;
  * a pure-Python scalar brute force (tests/bruteforce.py) in group form;
  * the pages' complexity formula and the 2.3% figure at 2048^2, the
    compression-ratio schedule (tests/golden/pages_facts.json).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import bruteforce as bf
import oracle as O
from synth_inputs import ALL_WORKLOADS, EXTRA_WORKLOADS, WORKLOADS, WORKLOAD_ORDER, Workload, make_all_weights, make_int_x, make_x, tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def _w(D, seed, scale=0.3, zero_k=False):
    g = np.random.default_rng(seed)
    w = {}
    for n in ("wq", "wk", "wv", "wo"):
        w[n] = g.standard_normal((D, D)) * scale
    for n in ("bq", "bk", "bv", "bo"):
        w[n] = g.standard_normal(D) * scale
    if zero_k:
        w["wk"][:] = 0
        w["bk"][:] = 0
    return w


def _torch_mha(xq, xkv, w, heads, mask=None):
    """Multi-head attention through torch's library routines, float64 CPU."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    q = torch.nn.functional.linear(t(xq), t(w["wq"]), t(w["bq"]))
    k = torch.nn.functional.linear(t(xkv), t(w["wk"]), t(w["bk"]))
    v = torch.nn.functional.linear(t(xkv), t(w["wv"]), t(w["bv"]))
    L, D = q.shape[-2], q.shape[-1]
    dh = D // heads
    sh = lambda a: a.reshape(*a.shape[:-1], heads, dh).transpose(-2, -3)
    o = torch.nn.functional.scaled_dot_product_attention(
        sh(q), sh(k), sh(v), attn_mask=None if mask is None else t(mask).bool())
    o = o.transpose(-2, -3).reshape(*q.shape[:-1], D)
    return torch.nn.functional.linear(o, t(w["wo"]), t(w["bo"])).numpy()


# ----------------------------------------------------------------------------- pool

@pytest.mark.parametrize("grid,p", [((1, 8, 8), (1, 2, 2)), ((1, 16, 16), (1, 4, 4)),
                                    ((1, 16, 16), (1, 8, 8)), ((2, 10, 15), (1, 5, 5)),
                                    ((4, 4, 6), (2, 2, 3)), ((1, 32, 32), (1, 16, 16))])
def test_pool_integer_inputs_exact(grid, p):
    """Integer tokens: the float32 nested-order mean is the correctly rounded
    quotient of the exact integer window sum (checked in rational arithmetic),
    and equals the float64 mean rounded to float32."""
    wl = tiny(H=grid[1], W=grid[2], F=grid[0], D=8, p=p)
    x = make_int_x(wl, seed=7)
    got = O.proxy_pool_f32(x, grid, p)
    ex = bf.pool([list(map(int, r)) for r in x[0]], grid, p)  # fsum of ints: exact
    P = p[0] * p[1] * p[2]
    F_, H, W = grid
    m = 0
    for T in range(F_ // p[0]):
        for I in range(H // p[1]):
            for J in range(W // p[2]):
                for c in range(x.shape[2]):
                    S = 0
                    for dt in range(p[0]):
                        for di in range(p[1]):
                            for dj in range(p[2]):
                                S += int(x[0, ((T * p[0] + dt) * H + I * p[1] + di) * W + J * p[2] + dj, c])
                    r = got[0, m, c]
                    exact = Fraction(S, P)
                    err = abs(Fraction(float(r)) - exact)
                    for nb in (np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(-np.inf))):
                        assert err <= abs(Fraction(float(nb)) - exact)
                    assert float(r) == float(np.float32(ex[m][c]))
                m += 1


def test_pool_f64_bruteforce_and_global_mean():
    wl = tiny(F=2, H=6, W=10, D=6, p=(2, 3, 5))
    x = make_x(wl, seed=11).astype(np.float64)
    got = O.proxy_pool(x, wl.grid, wl.p)
    ex = np.array(bf.pool(x[0].tolist(), wl.grid, wl.p))
    np.testing.assert_allclose(got[0], ex, rtol=0, atol=1e-14)
    # invariant: equal-size windows -> mean of proxies equals mean of tokens
    np.testing.assert_allclose(got.mean(axis=1), x.mean(axis=1), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- proxy selection (R-select)

@pytest.mark.parametrize("grid,p", [((4, 6, 9), (2, 3, 3)), ((1, 8, 8), (1, 4, 4)), ((3, 5, 7), (1, 1, 1)),
                                    ((2, 4, 6), (2, 4, 6))])
def test_select_is_a_strided_slice(grid, p):
    """Offset o = (dt*p_h + di)*p_w + dj selects the strided slice
    x[dt::p_t, di::p_h, dj::p_w] (numpy basic slicing), for every o; o = 0 /
    None is the top-left token of each window."""
    rng = np.random.default_rng(11)
    B, D = 2, 8
    x = rng.standard_normal((B, int(np.prod(grid)), D))
    xg = x.reshape(B, *grid, D)
    M = int(np.prod(O.proxy_grid(grid, p)))
    np.testing.assert_array_equal(O.proxy_select(x, grid, p),
                                  xg[:, ::p[0], ::p[1], ::p[2]].reshape(B, M, D))
    for dt in range(p[0]):
        for di in range(p[1]):
            for dj in range(p[2]):
                o = (dt * p[1] + di) * p[2] + dj
                got = O.proxy_select(x, grid, p, np.full((B, M), o))
                np.testing.assert_array_equal(got, xg[:, dt::p[0], di::p[1], dj::p[2]].reshape(B, M, D))


def test_select_offsets_per_window_bruteforce_and_mean():
    """Per-window offsets against a scalar loop over the grid (offsets taken
    modulo P, negative ones wrap); and the mean over all P offsets of the
    selections is the window average."""
    grid, p = (4, 6, 6), (2, 3, 2)
    rng = np.random.default_rng(12)
    B, D = 2, 4
    x = rng.standard_normal((B, int(np.prod(grid)), D))
    FT, HI, WJ = O.proxy_grid(grid, p)
    P = p[0] * p[1] * p[2]
    offs = rng.integers(-2 * P, 3 * P, size=(B, FT * HI * WJ))
    got = O.proxy_select(x, grid, p, offs)
    for b in range(B):
        for T in range(FT):
            for I in range(HI):
                for J in range(WJ):
                    m = (T * HI + I) * WJ + J
                    o = int(offs[b, m]) % P
                    dt, rem = divmod(o, p[1] * p[2])
                    di, dj = divmod(rem, p[2])
                    n = ((T * p[0] + dt) * grid[1] + I * p[1] + di) * grid[2] + J * p[2] + dj
                    np.testing.assert_array_equal(got[b, m], x[b, n])
    M = FT * HI * WJ
    allsel = sum(O.proxy_select(x, grid, p, np.full((B, M), o)) for o in range(P)) / P
    np.testing.assert_allclose(allsel, O.proxy_pool(x, grid, p), rtol=1e-12, atol=1e-12)


def test_block_with_selected_proxies_matches_bruteforce():
    """The block with top-left proxies equals the scalar brute force fed the
    same proxies: pool='select' changes only the proxy extraction."""
    wl = tiny("sel", B=1, F=2, H=4, W=4, D=8, heads=2, p=(2, 2, 2), win=(2, 4, 4), shift=(1, 2, 2))
    x = make_x(wl, seed=31)
    ws = make_all_weights(wl)
    got = O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads, pool="select")
    P = O.proxy_select(x, wl.grid, wl.p)
    np.testing.assert_array_equal(got["P"], P)
    P2 = O.proxy_sa(P, ws[0], wl.heads)
    x1 = O.proxy_xattn(x, P2, ws[1], wl.heads)
    np.testing.assert_allclose(got["x1"], x1, rtol=1e-12, atol=1e-12)
    # and the mean-pooled block differs (the variants are distinct)
    assert not np.allclose(O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads)["x3"], got["x3"])


# ----------------------------------------------------------------------------- text cross-attention and MLP

def test_gelu_tanh_matches_torch_and_identity():
    """The tanh form against torch's gelu(approximate='tanh') in float64 (a
    library routine), its odd-part identity gelu(x) - gelu(-x) = x, and its
    limits."""
    x = np.linspace(-12, 12, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, rtol=0, atol=1e-12)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu_tanh(np.array([12.0]))[0] - 12.0) < 1e-12
    assert abs(O.gelu_tanh(np.array([-12.0]))[0]) < 1e-12
    # not the erf form: they differ by ~1e-3 around |x| ~ 2
    erf = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(O.gelu_tanh(x) - erf)) > 1e-4


def test_mlp_closed_forms_and_scalar_loop():
    rng = np.random.default_rng(21)
    B, N, D, H = 2, 5, 8, 32
    x = rng.standard_normal((B, N, D))
    w = {"w1": rng.standard_normal((H, D)) * 0.3, "b1": rng.standard_normal(H) * 0.3,
         "w2": rng.standard_normal((D, H)) * 0.3, "b2": rng.standard_normal(D) * 0.3}
    # W1 = 0: the hidden layer is the constant gelu(b1)
    w0 = dict(w, w1=np.zeros((H, D)))
    const = w["w2"] @ O.gelu_tanh(w["b1"]) + w["b2"]
    np.testing.assert_allclose(O.mlp(x, w0), x + const, rtol=1e-12, atol=1e-12)
    # W2 = 0: only b2 and the residual remain
    np.testing.assert_allclose(O.mlp(x, dict(w, w2=np.zeros((D, H)))), x + w["b2"], rtol=1e-12, atol=1e-12)
    # scalar loop
    got = O.mlp(x, w, residual=False)
    for b in range(B):
        for n in range(N):
            h = [w["b1"][k] + sum(w["w1"][k, i] * x[b, n, i] for i in range(D)) for k in range(H)]
            g = [0.5 * v * (1 + math.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3))) for v in h]
            for j in range(D):
                y = w["b2"][j] + sum(w["w2"][j, k] * g[k] for k in range(H))
                assert abs(got[b, n, j] - y) < 1e-12


def test_text_xattn_is_mha_with_caption_keys():
    """Text cross-attention: uniform over the caption when W_k = 0 (closed
    form), and the block's x4/x5 follow x3 through text_xattn and mlp."""
    wl = tiny("txt", B=1, F=1, H=8, W=8, D=16, heads=2, p=(1, 2, 2), win=(1, 4, 4), shift=(0, 2, 2))
    x = make_x(wl, seed=41)
    rng = np.random.default_rng(42)
    text = rng.standard_normal((1, 7, wl.D))
    wt = make_all_weights(wl)[1]
    wz = dict(wt, wk=np.zeros_like(wt["wk"]), bk=np.zeros_like(wt["bk"]))
    v_mean = O.linear(text, wz["wv"], wz["bv"]).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(O.text_xattn(x, text, wz, wl.heads, residual=False),
                               np.broadcast_to(O.linear(v_mean, wz["wo"], wz["bo"]), x.shape), rtol=1e-12, atol=1e-12)
    wm = {"w1": rng.standard_normal((64, wl.D)) * 0.1, "b1": rng.standard_normal(64) * 0.1,
          "w2": rng.standard_normal((wl.D, 64)) * 0.1, "b2": rng.standard_normal(wl.D) * 0.1}
    ws = make_all_weights(wl)
    r = O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads, text=text, w_text=wt, w_mlp=wm)
    np.testing.assert_allclose(r["x4"], O.text_xattn(r["x3"], text, wt, wl.heads), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["x5"], O.mlp(r["x4"], wm), rtol=1e-12, atol=1e-12)


def test_pool_f32_close_to_f64():
    wl = tiny(H=32, W=32, D=64, p=(1, 8, 8))
    x = make_x(wl, seed=12)
    a = O.proxy_pool_f32(x, wl.grid, wl.p).astype(np.float64)
    b = O.proxy_pool(x, wl.grid, wl.p)
    # 64 float32 additions of |x| <= ~5: error far below 1e-5
    assert np.max(np.abs(a - b)) < 1e-5


def test_round_bf16_rne_matches_torch_cast():
    g = np.random.default_rng(3)
    vals = g.standard_normal(100000).astype(np.float32) * np.float32(10.0)
    # add exact ties: bf16 value + half ulp
    base = vals[:1000].view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    odd = ((base | np.uint32(0x10000)) | np.uint32(0x8000)).view(np.float32)
    allv = np.concatenate([vals, ties, odd, np.array([0.0, -0.0, 1e-40, 3.0e38], np.float32)])
    ours = O.round_bf16_rne(allv)
    ref = torch.from_numpy(allv).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------------------- attention

def test_attention_matches_torch_sdpa():
    g = np.random.default_rng(5)
    q, k, v = (g.standard_normal((3, 7, 24)) for _ in range(3))
    ours = O.attention(q, k[:, :5], v[:, :5], heads=3)
    t = lambda a: torch.from_numpy(a).reshape(3, -1, 3, 8).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k[:, :5]), t(v[:, :5]))
    ref = ref.transpose(1, 2).reshape(3, 7, 24).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)
    allow = g.random((3, 7, 5)) < 0.6
    allow[:, :, 0] = True
    ours = O.attention(q, k[:, :5], v[:, :5], heads=3, allow=allow)
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k[:, :5]), t(v[:, :5]), attn_mask=torch.from_numpy(allow)[:, None])
    np.testing.assert_allclose(ours, ref.transpose(1, 2).reshape(3, 7, 24).numpy(), rtol=1e-12, atol=1e-12)


def test_linear_matches_torch():
    g = np.random.default_rng(6)
    x, w, b = g.standard_normal((4, 3, 10)), g.standard_normal((6, 10)), g.standard_normal(6)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(O.linear(x, w, b), ref, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- GIIM

def test_proxy_p111_is_full_global_sa():
    """p = (1,1,1): every token is its own proxy, so the proxy SA is full
    global self-attention over all tokens."""
    wl = tiny(H=6, W=5, D=16, heads=2, p=(1, 1, 1))
    x = make_x(wl, seed=21).astype(np.float64)
    w = _w(16, 1)
    P = O.proxy_pool(x, wl.grid, wl.p)
    np.testing.assert_array_equal(P, x)
    got = O.proxy_sa(P, w, 2, residual=False)
    ref = _torch_mha(x[0], x[0], w, 2)
    np.testing.assert_allclose(got[0], ref, rtol=1e-10, atol=1e-12)


def test_one_proxy_closed_form():
    """p = whole grid: M = 1, softmax over one key is 1, so
    x1 = x + Lin(Lin(P'; Wv, bv); Wo, bo) for every token and
    P' = P + Lin(Lin(P; Wv, bv); Wo, bo)."""
    wl = tiny(F=2, H=4, W=4, D=8, heads=2, p=(2, 4, 4))
    x = make_x(wl, seed=22).astype(np.float64)
    w0, w1 = _w(8, 2), _w(8, 3)
    res = O.block(x, wl.grid, wl.p, (1, 2, 2), (0, 1, 1), [w0, w1, _w(8, 4), _w(8, 5)], 2)
    P = x.mean(axis=1, keepdims=True)
    P2 = P + ((P @ w0["wv"].T + w0["bv"]) @ w0["wo"].T + w0["bo"])
    np.testing.assert_allclose(res["P2"], P2, rtol=1e-12, atol=1e-12)
    x1 = x + ((P2 @ w1["wv"].T + w1["bv"]) @ w1["wo"].T + w1["bo"])
    np.testing.assert_allclose(res["x1"], x1, rtol=1e-12, atol=1e-12)


def test_xattn_uniform_when_wk_zero_and_permutation_invariant():
    g = np.random.default_rng(9)
    x = g.standard_normal((2, 12, 8))
    P2 = g.standard_normal((2, 5, 8))
    w = _w(8, 7, zero_k=True)
    got = O.proxy_xattn(x, P2, w, 2, residual=False)
    meanv = (P2 @ w["wv"].T + w["bv"]).mean(axis=1, keepdims=True)
    ref = np.broadcast_to(meanv @ w["wo"].T + w["bo"], got.shape)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    w = _w(8, 8)
    perm = g.permutation(5)
    a = O.proxy_xattn(x, P2, w, 2)
    b = O.proxy_xattn(x, P2[:, perm], w, 2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # residual is the input itself
    np.testing.assert_allclose(a - x, O.proxy_xattn(x, P2, w, 2, residual=False), atol=1e-13)


# ----------------------------------------------------------------------------- TCM

def test_wsa_whole_grid_is_full_sa():
    grid, win = (2, 4, 6), (2, 4, 6)
    g = np.random.default_rng(10)
    x = g.standard_normal((1, 48, 16))
    w = _w(16, 11)
    got = O.window_sa(x, grid, win, w, 2, residual=False)
    np.testing.assert_allclose(got[0], _torch_mha(x[0], x[0], w, 2), rtol=1e-10, atol=1e-12)
    # shift 0 on the same window is plain WSA, and equals full SA too
    got2 = O.shift_window_sa(x, grid, win, (0, 0, 0), w, 2, residual=False)
    np.testing.assert_array_equal(got, got2)


def test_wsa_one_token_window_closed_form():
    g = np.random.default_rng(12)
    x = g.standard_normal((1, 30, 8))
    w = _w(8, 13)
    got = O.window_sa(x, (1, 5, 6), (1, 1, 1), w, 2, residual=False)
    ref = (x @ w["wv"].T + w["bv"]) @ w["wo"].T + w["bo"]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _window_mean_ref(x, grid, win, shift, w):
    """W_k = 0 closed form: each real token gets Lin(mean of V over its group)."""
    F, H, W = grid
    D = x.shape[-1]
    out = np.zeros_like(x)
    for grp in bf._window_groups(grid, win, shift):
        vs = []
        for (t, i, j) in grp:
            tok = x[0, (t * H + i) * W + j] if (t < F and i < H and j < W) else np.zeros(D)
            vs.append(tok @ w["wv"].T + w["bv"])
        y = np.mean(vs, axis=0) @ w["wo"].T + w["bo"]
        for (t, i, j) in grp:
            if t < F and i < H and j < W:
                out[0, (t * H + i) * W + j] = y
    return out


@pytest.mark.parametrize("grid,win,shift", [((1, 8, 8), (1, 4, 4), (0, 2, 2)),
                                            ((1, 6, 10), (1, 4, 4), (0, 2, 2)),
                                            ((3, 6, 7), (2, 4, 4), (1, 2, 2)),
                                            ((2, 5, 9), (2, 4, 8), (1, 1, 3))])
def test_window_mean_of_v_pins_membership_and_pad(grid, win, shift):
    g = np.random.default_rng(14)
    N = int(np.prod(grid))
    x = g.standard_normal((1, N, 8))
    w = _w(8, 15, zero_k=True)
    got = O.window_sa(x, grid, win, w, 2, residual=False)
    np.testing.assert_allclose(got, _window_mean_ref(x, grid, win, (0, 0, 0), w), rtol=1e-12, atol=1e-12)
    got = O.shift_window_sa(x, grid, win, shift, w, 2, residual=False)
    np.testing.assert_allclose(got, _window_mean_ref(x, grid, win, shift, w), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("grid,win,shift", [((1, 8, 8), (1, 4, 4), (0, 2, 2)),
                                            ((1, 6, 10), (1, 4, 4), (0, 2, 2)),
                                            ((3, 6, 7), (2, 4, 4), (1, 2, 2)),
                                            ((2, 4, 8), (2, 4, 8), (1, 2, 3))])
def test_swsa_equals_group_form(grid, win, shift):
    """Roll + boundary mask + unroll equals attention inside the offset groups
    (independent implementation in tests/bruteforce.py)."""
    g = np.random.default_rng(16)
    N = int(np.prod(grid))
    x = g.standard_normal((1, N, 8))
    w = _w(8, 17)
    got = O.shift_window_sa(x, grid, win, shift, w, 2)
    ref = np.array(bf.window_attention(x[0].tolist(), grid, win, shift, w, 2))
    np.testing.assert_allclose(got[0], ref, rtol=1e-11, atol=1e-11)


def test_swsa_shift_zero_and_full_window_equal_wsa():
    g = np.random.default_rng(18)
    grid, win = (2, 8, 8), (2, 4, 4)
    x = g.standard_normal((2, 128, 8))
    w = _w(8, 19)
    wsa = O.window_sa(x, grid, win, w, 2)
    np.testing.assert_array_equal(wsa, O.shift_window_sa(x, grid, win, (0, 0, 0), w, 2))
    np.testing.assert_allclose(wsa, O.shift_window_sa(x, grid, win, (2, 4, 4), w, 2), rtol=1e-12, atol=1e-12)


def test_roll_matches_numpy_roll_and_inverts():
    g = np.random.default_rng(20)
    xg = g.standard_normal((2, 3, 5, 7, 4))
    for s in [(0, 0, 0), (1, 2, 3), (2, 4, 6)]:
        z = O.roll3d(xg, s)
        np.testing.assert_array_equal(z, np.roll(xg, shift=(-s[0], -s[1], -s[2]), axis=(1, 2, 3)))
        np.testing.assert_array_equal(O.roll3d(z, s, inverse=True), xg)


@pytest.mark.parametrize("grid,win,shift,sizes", [((1, 128, 128), (1, 8, 8), (0, 4, 4), [16, 32, 64]),
                                                  ((16, 30, 45), (2, 8, 8), (1, 4, 4), [16, 32, 64, 128])])
def test_mask_group_sizes(grid, win, shift, sizes):
    """Group sizes implied by the oracle's mask equal the group form's."""
    Lp = tuple(-(-a // b) * b for a, b in zip(grid, win))
    lab = O.region_labels(Lp, win, shift)
    wins = O.partition(lab[None, ..., None], win).reshape(-1, int(np.prod(win)))
    got = set()
    for r in wins:
        _, counts = np.unique(r, return_counts=True)
        got |= set(counts.tolist())
    assert sorted(got) == sizes == bf.group_sizes(grid, win, shift)


# ----------------------------------------------------------------------------- whole block

@pytest.mark.parametrize("B,grid,p,win,shift", [
    (1, (1, 8, 8), (1, 2, 2), (1, 4, 4), (0, 2, 2)),
    (2, (1, 6, 10), (1, 3, 5), (1, 4, 4), (0, 2, 2)),
    (1, (3, 6, 5), (1, 3, 5), (2, 4, 4), (1, 2, 2)),
])
def test_block_vs_scalar_bruteforce(B, grid, p, win, shift):
    g = np.random.default_rng(30)
    N = int(np.prod(grid))
    D, heads = 8, 2
    x = g.standard_normal((B, N, D))
    ws = [_w(D, 31 + a) for a in range(4)]
    got = O.block(x, grid, p, win, shift, ws, heads)["x3"]
    ref = np.array(bf.block(x.tolist(), grid, p, win, shift, ws, heads))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------- cost

def test_core_macs_match_pages_formula_and_2p3_percent():
    facts = json.load(open(GOLDEN))
    for name in WORKLOAD_ORDER:
        wl = WORKLOADS[name]
        c = O.count_core_macs(wl.grid, wl.p, wl.win, wl.D, B=wl.B)
        N, D, P = wl.N, wl.D, wl.p[0] * wl.p[1] * wl.p[2]
        Np = int(np.prod([-(-a // b) * b for a, b in zip(wl.grid, wl.win)]))
        wv = int(np.prod(wl.win))
        # complexity paragraph: 2N^2D/P^2 + 2N^2D/P, plus the window terms
        assert c["proxy_sa"] * P * P == wl.B * 2 * N * N * D
        assert c["xattn"] * P == wl.B * 2 * N * N * D
        assert c["wsa"] == c["swsa"] == wl.B * 2 * Np * wv * D
    wl = WORKLOADS["img2048"]
    c = O.count_core_macs(wl.grid, wl.p, wl.win, wl.D)
    share = Fraction(sum(c.values()), 2 * wl.N * wl.N * wl.D)
    pct = float(share) * 100
    assert abs(pct - 2.368) < 1e-3
    assert f"{math.floor(pct * 10) / 10:.1f}" == facts["complexity_share_2048_percent"]["value"]


def test_core_macs_counted_from_the_oracles_own_products(monkeypatch):
    """The complexity paragraph's formula (2N^2D/P^2 + 2N^2D/P for GIIM, plus
    the two window terms) against multiply-accumulates counted from the
    operand shapes of the attention products the oracle actually runs inside
    block() on the 2048^2 grid (narrow D: the count is linear in D), and the
    2.3% share computed from those counts."""
    facts = json.load(open(GOLDEN))
    from oracle import ptdit_oracle as PO
    real = PO.attention
    calls = []

    def counting(q, k, v, heads, allow=None):
        lq = int(np.prod(q.shape[:-1]))          # every query row of the call
        lk = k.shape[-2]                         # keys per query row
        calls.append(2 * lq * lk * q.shape[-1])  # Q K^T and A V
        return real(q, k, v, heads, allow)

    monkeypatch.setattr(PO, "attention", counting)
    wl = WORKLOADS["img2048"]
    D, heads = 16, 2
    g = np.random.default_rng(5)
    x = g.standard_normal((1, wl.N, D))
    ws = [_w(D, 90 + a, scale=0.1) for a in range(4)]
    O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, heads)
    assert len(calls) == 4                      # proxy SA, cross, WSA, SWSA
    N, P, L = wl.N, int(np.prod(wl.p)), int(np.prod(wl.win))
    assert calls[0] == 2 * N * N * D // (P * P)
    assert calls[1] == 2 * N * N * D // P
    assert calls[2] == calls[3] == 2 * N * L * D
    share = Fraction(sum(calls), 2 * N * N * D)
    pct = float(share) * 100
    assert abs(pct - 2.368) < 1e-3
    assert f"{math.floor(pct * 10) / 10:.1f}" == facts["complexity_share_2048_percent"]["value"]
    # a planted slip (the cross-attention counted with the queries and keys
    # swapped, i.e. keys = tokens) moves the share far from the page's figure
    assert abs(float(Fraction(calls[0] + 2 * N * N * D + calls[2] + calls[3], 2 * N * N * D)) * 100 - 2.3) > 50


def test_oracle_float32_mode_tracks_float64():
    """precision(np.float32) runs the same steps in float32 (the CPU baseline's
    fp32 oracle): its block output is float32 and within float32 rounding of
    the float64 oracle, which is pinned by every other test here."""
    wl = WORKLOADS["img256_f32"]
    x = make_x(wl)
    ws = make_all_weights(wl)
    ref = O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads)["x3"]
    with O.precision(np.float32):
        got = O.block(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads)["x3"]
    assert got.dtype == np.float32
    assert O.block(x[:, :64], (1, 8, 8), (1, 2, 2), (1, 8, 8), (0, 4, 4), ws, wl.heads)["x3"].dtype == np.float64
    d = got.astype(np.float64) - ref
    assert np.linalg.norm(d) / np.linalg.norm(ref) < 1e-5
    assert np.abs(d).max() < 1e-4


def test_compression_schedule_keeps_proxy_count():
    facts = json.load(open(GOLDEN))
    for down in (8, 16):  # any fixed total latent downsampling factor
        counts = set()
        for res, p in facts["compression_ratios_image"]["value"]:
            grid = (1, res // down, res // down)
            counts.add(int(np.prod(O.proxy_grid(grid, p))))
        assert len(counts) == 1
    for name in WORKLOAD_ORDER[:3] + ["img4096"]:
        wl = WORKLOADS[name]
        assert wl.M == 256


def test_video_workloads_follow_pages_ratios():
    """The extra video workloads compress time by the pages' fixed p_f and
    space by the image schedule's ratio for their view size (512^2 views ->
    32x32 latent tokens under 8x VAE and 2x2 patches)."""
    facts = json.load(open(GOLDEN))
    pf = facts["video_temporal_ratio"]["value"]
    spatial = {res // 16: tuple(p[1:]) for res, p in facts["compression_ratios_image"]["value"]}
    for name, wl in EXTRA_WORKLOADS.items():
        assert wl.p[0] == pf, name
        assert wl.F % pf == 0 and wl.H % wl.p[1] == 0 and wl.W % wl.p[2] == 0, name
        if wl.H == wl.W:
            assert tuple(wl.p[1:]) == spatial[wl.H], name
    # the three proxy counts
    assert [EXTRA_WORKLOADS[n].M for n in ("video16x30x45_pf4", "mview24x32x32", "video72x32x32")] == \
        [4 * 6 * 9, 6 * 8 * 8, 18 * 8 * 8]
    # cost model holds for every workload (pages' complexity paragraph)
    for name in ALL_WORKLOADS:
        wl = WORKLOADS[name]
        c = O.count_core_macs(wl.grid, wl.p, wl.win, wl.D, B=wl.B)
        P = wl.p[0] * wl.p[1] * wl.p[2]
        assert c["xattn"] * P == wl.B * 2 * wl.N * wl.N * wl.D


def test_projection_macs_img2048():
    wl = WORKLOADS["img2048"]
    pm = O.count_projection_macs(wl.grid, wl.p, wl.win, wl.D)
    cm = O.count_core_macs(wl.grid, wl.p, wl.win, wl.D)
    gf = 2 * (sum(pm.values()) + sum(cm.values())) / 1e9
    assert abs(gf - 468.24) < 0.01
