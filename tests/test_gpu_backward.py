"""GPU parity of the backward pass (through the C ABI) against the float64
backward oracle (oracle/ptdit_backward.py, itself pinned to finite
differences, torch autograd and adjoint identities): the attention cores, the
window average, the roll and the projections' gradients.

Bar: max-abs 2e-2 and relative-L2 1e-2 for every gradient (tests/gpu_util.py);
the non-accumulating pooling backward is an IEEE division by P and is compared
bit for bit with the float64 result rounded to float32 (exact: a float64
quotient rounded to float32 is the correctly rounded float32 quotient).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_close, dev, host
from synth_inputs import make_attn_grad_inputs, round_bf16

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_attention_pt_amd as P
    P.load()
    return P


def tok(a):
    """[B, heads, L, dh] -> token-major [B, L, heads*dh]."""
    B, h, L, dh = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B, L, h * dh)


# ----------------------------------------------------------------------------- window core

WIN_CASES = {
    # grid (B, F, H, W), D, heads, window, shift, dtype, score scale
    "img_pad_shift": ((1, 1, 20, 36), 1152, 16, (1, 8, 8), (0, 4, 4), "bf16", 1.0),
    "img_batch2_noshift": ((2, 1, 16, 24), 1152, 16, (1, 8, 8), (0, 0, 0), "bf16", 1.0),
    "video_pad_shift": ((1, 3, 10, 12), 1152, 16, (2, 8, 8), (1, 4, 4), "bf16", 1.0),
    "dh64_shift": ((1, 1, 16, 16), 1024, 16, (1, 8, 8), (0, 4, 4), "bf16", 1.0),
    "f32_video_pad": ((1, 3, 10, 12), 1152, 16, (2, 8, 8), (1, 4, 4), "f32", 1.0),
    "peaked_shift": ((1, 1, 24, 24), 1152, 16, (1, 8, 8), (0, 4, 4), "bf16", 1.7),
    "small_window_pad": ((1, 2, 5, 7), 576, 8, (1, 4, 4), (0, 2, 2), "bf16", 1.0),
}


@pytest.mark.parametrize("name", list(WIN_CASES))
def test_window_attn_bwd_vs_oracle(P, name):
    (B, F, H, W), D, heads, win, shift, dt, scale = WIN_CASES[name]
    dh, N = D // heads, F * H * W
    announce(f"window bwd {name} grid={(B, F, H, W)} D={D} win={win} shift={shift} {dt}")
    q, k, v, do = make_attn_grad_inputs(B, heads, N, N, dh, seed=300 + len(name), scale=scale, dtype=dt)
    g = np.random.Generator(np.random.PCG64(400 + len(name)))
    bias = g.standard_normal(3 * D).astype(np.float32) * 0.5
    if dt == "bf16":
        bias = round_bf16(bias)
    prec = BF16 if dt == "bf16" else F32
    qkv = np.stack([q, k, v], axis=1)                        # [B, 3, heads, N, dh]
    dqkv, dbkv = P.window_attn_bwd(dev(qkv, prec), dev(do, prec), (B, F, H, W, D, heads), win, shift,
                                   b_qkv=dev(bias, prec))
    torch.cuda.synchronize()
    dqkv = host(dqkv)
    rq, rk, rv, rkp, rvp = O.window_core_bwd(tok(q), tok(k), tok(v), do, (F, H, W), win, shift, heads,
                                            bias[D:2 * D], bias[2 * D:])
    assert_close(tok(dqkv[:, 0]), rq, "dQ")
    assert_close(tok(dqkv[:, 1]), rk, "dK")
    assert_close(tok(dqkv[:, 2]), rv, "dV")
    assert_close(host(dbkv), np.stack([rkp, rvp]), "d pad k/v")


def test_window_attn_bwd_full_size_sampled_windows(P):
    # the 2048^2 image grid (128 x 128 tokens, 16 heads of 72) with the TCM
    # shift: the whole backward on the GPU, seven windows (the first, the
    # wrap-around corner under the boundary mask, five drawn) by the oracle
    B, F, H, W, D, heads = 1, 1, 128, 128, 1152, 16
    win, shift = (1, 8, 8), (0, 4, 4)
    dh, N = D // heads, F * H * W
    announce("window bwd full size 1x128x128 shift (0,4,4)")
    q, k, v, do = make_attn_grad_inputs(B, heads, N, N, dh, seed=350)
    qkv = np.stack([q, k, v], axis=1)
    dqkv, _ = P.window_attn_bwd(dev(qkv, BF16), dev(do, BF16), (B, F, H, W, D, heads), win, shift)
    torch.cuda.synchronize()
    dqkv = host(dqkv)
    # token ids and labels of every window slot, from the oracle's own roll / partition
    ids = np.arange(N, dtype=np.float64).reshape(1, F, H, W, 1)
    slots = O.partition(O.roll3d(ids, shift), win).reshape(-1, 64).astype(np.int64)
    labs = O.partition(O.region_labels((F, H, W), win, shift)[None, ..., None], win).reshape(-1, 64)
    g = np.random.Generator(np.random.PCG64(351))
    picks = [0, slots.shape[0] - 1] + list(g.choice(slots.shape[0], 5, replace=False))
    qt, kt, vt = tok(q)[0], tok(k)[0], tok(v)[0]
    for w in picks:
        t = slots[w]
        allow = labs[w][:, None] == labs[w][None, :]
        rq, rk, rv = O.attention_bwd(qt[t], kt[t], vt[t], do[0][t], heads, allow)
        assert_close(tok(dqkv[:, 0])[0][t], rq, f"dQ window {w}")
        assert_close(tok(dqkv[:, 1])[0][t], rk, f"dK window {w}")
        assert_close(tok(dqkv[:, 2])[0][t], rv, f"dV window {w}")


# ----------------------------------------------------------------------------- dense core

DENSE_CASES = {
    # B, heads, Nq, Nk, dh, layout ("qkv": views of one [B,3,heads,M,dh] buffer,
    # "q+kv": q alone, k/v views of [B,2,heads,M,dh]), dtype, score scale
    "proxy_sa_fused": (2, 16, 256, 256, 72, "qkv", "bf16", 1.0),
    "xattn_chunks_ragged": (1, 16, 2400, 150, 72, "q+kv", "bf16", 1.0),
    "xattn_peaked": (1, 16, 1100, 256, 72, "q+kv", "bf16", 1.7),
    "dh64": (2, 16, 300, 64, 64, "q+kv", "bf16", 1.0),
    "f32": (1, 8, 1500, 96, 72, "q+kv", "f32", 1.0),
    "one_key": (1, 4, 70, 1, 72, "q+kv", "bf16", 1.0),
    # more than 256 keys: the vector-ALU query-major kernel with the
    # matrix-core key-major kernel (statistics handed between them)
    "many_keys": (1, 16, 1100, 600, 72, "q+kv", "bf16", 1.0),
    "batch2_chunks": (2, 16, 2100, 256, 72, "q+kv", "bf16", 1.0),
}


@pytest.mark.parametrize("name", list(DENSE_CASES))
def test_attn_bwd_vs_oracle(P, name):
    B, heads, Nq, Nk, dh, layout, dt, scale = DENSE_CASES[name]
    announce(f"dense bwd {name} B={B} heads={heads} Nq={Nq} Nk={Nk} dh={dh} {layout} {dt}")
    q, k, v, do = make_attn_grad_inputs(B, heads, Nq, Nk, dh, seed=500 + len(name), scale=scale, dtype=dt)
    prec = BF16 if dt == "bf16" else F32
    if layout == "qkv":
        buf = dev(np.stack([q, k, v], axis=1), prec)         # Nq == Nk
        qd, kd, vd = buf[:, 0], buf[:, 1], buf[:, 2]
    else:
        qd = dev(q, prec)
        kv = dev(np.stack([k, v], axis=1), prec)
        kd, vd = kv[:, 0], kv[:, 1]
    dq, dk, dv = P.attn_bwd(qd, kd, vd, dev(do, prec))
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_bwd(tok(q), tok(k), tok(v), do, heads)
    if Nk == 1:
        # one key: every weight is 1, so dQ = dK = 0 exactly (a relative error
        # means nothing there; the kernel's dQ = dA k - D k leaves one rounding
        # of dA k) and dV is the sum of dO
        assert np.all(rq == 0) and np.all(rk == 0)
        assert np.abs(host(dq)).max() <= 1e-5 and np.abs(host(dk)).max() <= 1e-5
    else:
        assert_close(tok(host(dq)), rq, "dQ")
        assert_close(tok(host(dk)), rk, "dK")
    assert_close(tok(host(dv)), rv, "dV")


def test_attn_bwd_full_size_cross_attention(P):
    # cross-attention at 2048^2: 16384 token queries, 256 proxies, 16 heads;
    # the oracle takes two heads whole (dK, dV sum over every query)
    B, heads, Nq, Nk, dh = 1, 16, 16384, 256, 72
    announce("dense bwd full size Nq=16384 Nk=256")
    q, k, v, do = make_attn_grad_inputs(B, heads, Nq, Nk, dh, seed=550)
    kv = dev(np.stack([k, v], axis=1), BF16)
    dq, dk, dv = P.attn_bwd(dev(q, BF16), kv[:, 0], kv[:, 1], dev(do, BF16))
    torch.cuda.synchronize()
    dq, dk, dv = host(dq), host(dk), host(dv)
    for h in (0, heads - 1):
        sl = slice(h * dh, (h + 1) * dh)
        rq, rk, rv = O.attention_bwd(q[0, h], k[0, h], v[0, h], do[0][:, sl], 1)
        assert_close(dq[0, h], rq, f"dQ head {h}")
        assert_close(dk[0, h], rk, f"dK head {h}")
        assert_close(dv[0, h], rv, f"dV head {h}")


# ----------------------------------------------------------------------------- pooling

POOL_CASES = [
    ((1, 1, 16, 16), 1152, (1, 4, 4)),
    ((2, 4, 6, 9), 64, (2, 3, 3)),
    ((1, 1, 128, 128), 1152, (1, 8, 8)),
    ((1, 3, 5, 7), 2400, (3, 5, 7)),   # 105 rows (a ragged 8-row group), two column passes
    ((3, 1, 3, 5), 8, (1, 3, 5)),      # 45 rows over three batches, two columns
]


@pytest.mark.parametrize("case", POOL_CASES)
def test_proxy_pool_bwd_vs_oracle(P, case):
    (B, F, H, W), D, p = case
    announce(f"pool bwd grid={(B, F, H, W)} D={D} p={p}")
    M = (F // p[0]) * (H // p[1]) * (W // p[2])
    g = np.random.Generator(np.random.PCG64(600 + D))
    dP = g.standard_normal((B, M, D)).astype(np.float32)
    grid = (B, F, H, W, D, 16)
    ref = O.proxy_pool_bwd(dP, (F, H, W), p)
    got = host(P.proxy_pool_bwd(dev(dP, F32), grid, p))
    np.testing.assert_array_equal(got, ref.astype(np.float32).astype(np.float64))
    base = g.standard_normal((B, F * H * W, D)).astype(np.float32)
    acc = host(P.proxy_pool_bwd(dev(dP, F32), grid, p, d_x=dev(base, F32), accumulate=True))
    np.testing.assert_allclose(acc, base + ref, rtol=1e-6, atol=1e-6)


def test_roll_bwd_is_the_inverse_roll(P):
    # the roll's gradient is the inverse roll (pinned on the CPU); on the GPU
    # the inverse roll of the forward roll is the identity, bit for bit
    g = np.random.Generator(np.random.PCG64(650))
    grid = (2, 3, 10, 12, 64, 1)
    x = dev(g.standard_normal((2, 360, 64)).astype(np.float32), F32)
    y = P.roll3d(P.roll3d(x, grid, (1, 4, 4)), grid, (1, 4, 4), inverse=True)
    assert torch.equal(x, y)


# ----------------------------------------------------------------------------- projections

LIN_CASES = [
    # rows, d_in, d_out, x dtype, d_y dtype
    (2400, 1152, 1152, "bf16", "bf16"),
    (2400, 1152, 1152, "bf16", "f32"),
    (300, 1152, 3456, "bf16", "bf16"),
    (1, 8, 16, "bf16", "f32"),
    (777, 64, 200, "f32", "f32"),
    (16384, 1152, 1152, "bf16", "f32"),   # the 2048^2 output projection
]


@pytest.mark.parametrize("case", LIN_CASES)
def test_linear_bwd_vs_oracle(P, case):
    rows, d_in, d_out, xdt, ydt = case
    announce(f"linear bwd rows={rows} d_in={d_in} d_out={d_out} x {xdt} dy {ydt}")
    g = np.random.Generator(np.random.PCG64(700 + rows + d_out))
    x = g.standard_normal((rows, d_in)).astype(np.float32)
    w = round_bf16(g.standard_normal((d_out, d_in)).astype(np.float32) * 0.02)
    dy = g.standard_normal((rows, d_out)).astype(np.float32)
    if xdt == "bf16":
        x = round_bf16(x)
    if ydt == "bf16":
        dy = round_bf16(dy)
    dx, dw, db = P.linear_bwd(dev(x, BF16 if xdt == "bf16" else F32), dev(w, BF16),
                              dev(dy, BF16 if ydt == "bf16" else F32))
    torch.cuda.synchronize()
    rx, rw, rb = O.linear_bwd(x, w, dy)
    # the products take bf16 operands (an fp32 d_y or x is rounded, relative
    # error 2^-9 per term): d_x sums d_out terms of size |w| ~ 0.02; d_w and d_b
    # sum `rows` terms of size ~1 and grow as sqrt(rows), so they are compared
    # after division by sqrt(rows)
    assert_close(host(dx), rx, "dX")
    n = np.sqrt(rows)
    assert_close(host(dw) / n, rw / n, "dW / sqrt(rows)")
    assert_close(host(db) / n, rb / n, "db / sqrt(rows)")
