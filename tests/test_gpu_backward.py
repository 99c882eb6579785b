"""GPU parity of the backward pass (through the C ABI) against the float64
backward oracle (oracle/ptdit_backward.py, itself pinned to finite
differences, torch autograd and adjoint identities): the attention cores, the
window average, the roll and the projections' gradients.

Bar (tests/gpu_util.py, grad_bar): relative-L2 1e-2 and max-abs 2e-2 scaled by
max(1, largest magnitude of the reference gradient) for every gradient;
the non-accumulating pooling backward is an IEEE division by P and is compared
bit for bit with the float64 result rounded to float32 (exact: a float64
quotient rounded to float32 is the correctly rounded float32 quotient).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_grad_close, dev, host
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
    # 64-token windows on the matrix-core kernel with a pad (4) that differs
    # from the shift (2): pad slots share a mask region with real tokens, so
    # their key/value gradients (d b_k, d b_v) are nonzero
    "img_pad_ne_shift": ((1, 1, 20, 36), 1152, 16, (1, 8, 8), (0, 2, 2), "bf16", 1.0),
    # the same over 20 padded windows of a 60 x 100 grid (the bias sums add
    # the pad slots of every one of them)
    "img_many_pad_windows": ((1, 1, 60, 100), 1152, 16, (1, 8, 8), (0, 2, 2), "bf16", 1.0),
    # 128-token video windows (2 x 8 x 8) on the matrix-core kernel: head width
    # 64; batch 2 without a shift; a pad (1 frame, 4 rows, 4 columns) that
    # differs from the shift (1, 2, 2), so pad slots are visible
    "video128_dh64": ((1, 4, 16, 16), 1024, 16, (2, 8, 8), (1, 4, 4), "bf16", 1.0),
    "video128_batch2_noshift": ((2, 4, 16, 16), 1152, 16, (2, 8, 8), (0, 0, 0), "bf16", 1.0),
    "video128_pad_ne_shift": ((1, 3, 20, 36), 1152, 16, (2, 8, 8), (1, 2, 2), "bf16", 1.0),
    "video128_peaked": ((1, 4, 16, 16), 1152, 16, (2, 8, 8), (1, 4, 4), "bf16", 1.7),
    # 96-token windows (1 x 8 x 12): slots 96..127 of the 128-slot kernel are
    # empty
    "window96_shift": ((1, 1, 16, 24), 1152, 16, (1, 8, 12), (0, 4, 6), "bf16", 1.0),
}

# cases whose pad slots are visible to real queries (their pad gradients must
# be nonzero, so the bias-sum path is exercised)
PAD_VISIBLE = {"img_pad_ne_shift", "img_many_pad_windows", "small_window_pad", "video_pad_shift",
               "f32_video_pad", "video128_pad_ne_shift"}


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
    assert_grad_close(tok(dqkv[:, 0]), rq, "dQ")
    assert_grad_close(tok(dqkv[:, 1]), rk, "dK")
    assert_grad_close(tok(dqkv[:, 2]), rv, "dV")
    assert_grad_close(host(dbkv), np.stack([rkp, rvp]), "d pad k/v")
    if name in PAD_VISIBLE:
        assert np.abs(rkp).max() > 1e-3 and np.abs(rvp).max() > 1e-3, "pad gradients should be nonzero here"


@pytest.mark.parametrize("name", ["img_batch2_noshift", "dh64_shift", "img_pad_shift"])
def test_window_attn_bwd_without_pad_buffer(P, name):
    """pad_grad=False passes no pad-slot buffer: where the window divides the
    grid the gradients equal those of a call with one, bit for bit, and no
    buffer comes back; where it does not, the library refuses the call."""
    from diffusion_transformer_attention_pt_amd import _lib
    (B, F, H, W), D, heads, win, shift, dt, scale = WIN_CASES[name]
    dh, N = D // heads, F * H * W
    announce(f"window bwd without pad buffer {name}")
    q, k, v, do = make_attn_grad_inputs(B, heads, N, N, dh, seed=350 + len(name), scale=scale, dtype=dt)
    qkv = dev(np.stack([q, k, v], axis=1), BF16)
    grid = (B, F, H, W, D, heads)
    divides = all(gs % ws == 0 for gs, ws in zip((F, H, W), win))
    if not divides:
        with pytest.raises(_lib.PtditError):
            _lib.window_attn_bwd(qkv, dev(do, BF16), grid, win, shift, tokens=True, pad_grad=False)
        return
    d_ref, db_ref = _lib.window_attn_bwd(qkv, dev(do, BF16), grid, win, shift, tokens=True)
    d_new, db_new = _lib.window_attn_bwd(qkv, dev(do, BF16), grid, win, shift, tokens=True, pad_grad=False)
    torch.cuda.synchronize()
    assert db_new is None
    assert torch.equal(d_new, d_ref)
    assert not host(db_ref).any()


@pytest.mark.parametrize("name", ["img_pad_ne_shift", "video128_pad_ne_shift", "f32_video_pad", "dh64_shift"])
def test_window_attn_bwd_tokens_layout(P, name):
    """ptdit_window_attn_bwd_tokens writes the same values as
    ptdit_window_attn_bwd, token-major: bit for bit equal to the head-major
    result after the layout change, and with bf16 gradients, to that result
    rounded to bf16; the pad-slot bias gradients agree to the order of their
    atomic additions."""
    from diffusion_transformer_attention_pt_amd import _lib
    (B, F, H, W), D, heads, win, shift, dt, scale = WIN_CASES[name]
    dh, N = D // heads, F * H * W
    announce(f"window bwd tokens layout {name}")
    q, k, v, do = make_attn_grad_inputs(B, heads, N, N, dh, seed=320 + len(name), scale=scale, dtype=dt)
    g = np.random.Generator(np.random.PCG64(420 + len(name)))
    bias = g.standard_normal(3 * D).astype(np.float32) * 0.5
    prec = BF16 if dt == "bf16" else F32
    if dt == "bf16":
        bias = round_bf16(bias)
    qkv = dev(np.stack([q, k, v], axis=1), prec)
    dqkv_h, db_h = P.window_attn_bwd(qkv, dev(do, prec), (B, F, H, W, D, heads), win, shift, b_qkv=dev(bias, prec))
    dqkv_t, db_t = _lib.window_attn_bwd(qkv, dev(do, prec), (B, F, H, W, D, heads), win, shift,
                                        b_qkv=dev(bias, prec), tokens=True)
    torch.cuda.synchronize()
    assert tuple(dqkv_t.shape) == (B, N, 3 * D)
    assert torch.equal(dqkv_t, _lib.heads_to_tokens(dqkv_h))
    np.testing.assert_allclose(host(db_t), host(db_h), rtol=1e-5, atol=1e-5)
    if dt == "bf16":
        # bf16 gradients: the fp32 values rounded to nearest even, bit for bit
        d16 = torch.empty(B, N, 3 * D, dtype=BF16, device="cuda")
        _, db16 = _lib.window_attn_bwd(qkv, dev(do, prec), (B, F, H, W, D, heads), win, shift,
                                       b_qkv=dev(bias, prec), tokens=True, d_qkv=d16)
        torch.cuda.synchronize()
        assert torch.equal(d16.view(torch.int16), dqkv_t.to(BF16).view(torch.int16))
        np.testing.assert_allclose(host(db16), host(db_h), rtol=1e-5, atol=1e-5)
    else:
        with pytest.raises(_lib.PtditError):   # bf16 gradients only from bf16 inputs
            _lib.window_attn_bwd(qkv, dev(do, prec), (B, F, H, W, D, heads), win, shift, b_qkv=dev(bias, prec),
                                 tokens=True, d_qkv=torch.empty(B, N, 3 * D, dtype=BF16, device="cuda"))


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
        assert_grad_close(tok(dqkv[:, 0])[0][t], rq, f"dQ window {w}")
        assert_grad_close(tok(dqkv[:, 1])[0][t], rk, f"dK window {w}")
        assert_grad_close(tok(dqkv[:, 2])[0][t], rv, f"dV window {w}")


def test_window_attn_bwd_video_full_size_sampled_windows(P):
    # the 16 x 30 x 45 video grid (padded to 16 x 32 x 48 for 2 x 8 x 8
    # windows, 128 tokens) with the temporal shift (1, 4, 4): the whole backward
    # on the matrix-core 128-token kernel, six windows by the oracle (the
    # first, the wrap-around corner, four drawn)
    B, F, H, W, D, heads = 1, 16, 30, 45, 1152, 16
    win, shift = (2, 8, 8), (1, 4, 4)
    dh, N = D // heads, F * H * W
    announce("window bwd full size video 16x30x45 win (2,8,8) shift (1,4,4)")
    q, k, v, do = make_attn_grad_inputs(B, heads, N, N, dh, seed=352)
    g = np.random.Generator(np.random.PCG64(353))
    bias = round_bf16(g.standard_normal(3 * D).astype(np.float32) * 0.5)
    qkv = np.stack([q, k, v], axis=1)
    dqkv, dbkv = P.window_attn_bwd(dev(qkv, BF16), dev(do, BF16), (B, F, H, W, D, heads), win, shift,
                                   b_qkv=dev(bias, BF16))
    torch.cuda.synchronize()
    dqkv = host(dqkv)
    grid_p = tuple(-(-n // w) * w for n, w in zip((F, H, W), win))
    # slot -> token (or pad) of every window, from the oracle's own pad, roll and partition
    ids = np.full((1,) + grid_p + (1,), -1.0)
    ids[0, :F, :H, :W, 0] = np.arange(N, dtype=np.float64).reshape(F, H, W)
    slots = O.partition(O.roll3d(ids, shift), win).reshape(-1, 128).astype(np.int64)
    labs = O.partition(O.region_labels(grid_p, win, shift)[None, ..., None], win).reshape(-1, 128)
    picks = [0, slots.shape[0] - 1] + list(g.choice(slots.shape[0], 4, replace=False))
    qt, kt, vt = tok(q)[0], tok(k)[0], tok(v)[0]
    bk, bv = bias[D:2 * D], bias[2 * D:]
    for w in picks:
        t = slots[w]
        real = t >= 0
        allow = labs[w][:, None] == labs[w][None, :]
        kw = np.where(real[:, None], kt[np.maximum(t, 0)], bk[None, :])      # pad keys / values are the biases
        vw = np.where(real[:, None], vt[np.maximum(t, 0)], bv[None, :])
        qw = np.where(real[:, None], qt[np.maximum(t, 0)], 0.0)
        dow = np.where(real[:, None], do[0][np.maximum(t, 0)], 0.0)
        rq, rk, rv = O.attention_bwd(qw, kw, vw, dow, heads, allow)
        tr = t[real]
        assert_grad_close(tok(dqkv[:, 0])[0][tr], rq[real], f"dQ window {w}")
        assert_grad_close(tok(dqkv[:, 1])[0][tr], rk[real], f"dK window {w}")
        assert_grad_close(tok(dqkv[:, 2])[0][tr], rv[real], f"dV window {w}")


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
    # more than 256 keys: the streamed query-major kernel (keys in chunks of
    # 256, two passes) with the key-major kernel (statistics handed between
    # them); 600 keys end in a ragged half chunk
    "many_keys": (1, 16, 1100, 600, 72, "q+kv", "bf16", 1.0),
    # the 16 x 30 x 45 video's proxy self-attention (864 proxies) and its
    # cross-attention on a slice of the queries; 1152 proxies of the long video
    # (72 x 32 x 32, proxy window 2 x 4 x 4) with peaked scores; head width 64
    "video_proxy_sa_864": (1, 16, 864, 864, 72, "qkv", "bf16", 1.0),
    "video_xattn_864": (1, 16, 3000, 864, 72, "q+kv", "bf16", 1.0),
    "long_video_1152_peaked": (1, 16, 1152, 1152, 72, "qkv", "bf16", 1.7),
    "many_keys_dh64": (1, 16, 700, 300, 64, "q+kv", "bf16", 1.0),
    # 257 keys: one key past a whole chunk (a second chunk of one key)
    "keys_257": (1, 8, 500, 257, 72, "q+kv", "bf16", 1.0),
    "batch2_chunks": (2, 16, 2100, 256, 72, "q+kv", "bf16", 1.0),
    # few keys against thousands of queries: every dK / dV row sums
    # thousands of products (the randomized sweep's largest absolute errors)
    "few_keys_3000q": (1, 16, 3000, 16, 72, "q+kv", "bf16", 1.0),
    "eight_keys_4096q": (1, 16, 4096, 8, 72, "q+kv", "bf16", 1.0),
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
        assert_grad_close(tok(host(dq)), rq, "dQ")
        assert_grad_close(tok(host(dk)), rk, "dK")
    assert_grad_close(tok(host(dv)), rv, "dV")


@pytest.mark.parametrize("name", ["xattn_chunks_ragged", "many_keys", "dh64", "f32"])
def test_attn_bwd_tokens_layout(P, name):
    """ptdit_attn_bwd_tokens: dQ token-major, bit for bit the head-major dQ
    of ptdit_attn_bwd after the layout change, and with bf16 gradients that
    result rounded to bf16; dK and dV unchanged (fp32 inputs: bf16 gradients
    are refused)."""
    from diffusion_transformer_attention_pt_amd import _lib
    B, heads, Nq, Nk, dh, layout, dt, scale = DENSE_CASES[name]
    announce(f"dense bwd tokens layout {name}")
    q, k, v, do = make_attn_grad_inputs(B, heads, Nq, Nk, dh, seed=560 + len(name), scale=scale, dtype=dt)
    prec = BF16 if dt == "bf16" else F32
    qd = dev(q, prec)
    kv = dev(np.stack([k, v], axis=1), prec)
    dd = dev(do, prec)
    dq, dk, dv = P.attn_bwd(qd, kv[:, 0], kv[:, 1], dd)
    dq_t, dk_t, dv_t = _lib.attn_bwd(qd, kv[:, 0], kv[:, 1], dd, dq_tokens=True)
    torch.cuda.synchronize()
    assert tuple(dq_t.shape) == (B, Nq, heads * dh)
    assert torch.equal(dq_t, dq.transpose(1, 2).reshape(B, Nq, heads * dh))
    assert torch.equal(dk_t, dk) and torch.equal(dv_t, dv)
    d16 = torch.empty(B, Nq, heads * dh, dtype=BF16, device="cuda")
    if dt == "bf16":
        _lib.attn_bwd(qd, kv[:, 0], kv[:, 1], dd, dq=d16, dq_tokens=True)
        torch.cuda.synchronize()
        assert torch.equal(d16.view(torch.int16), dq_t.to(BF16).view(torch.int16))
    else:
        with pytest.raises(_lib.PtditError):
            _lib.attn_bwd(qd, kv[:, 0], kv[:, 1], dd, dq=d16, dq_tokens=True)


def test_linear_bwd_token_major_matches_transposed(P):
    """The weight gradient from token-major bf16 operands equals, bit for bit,
    the one from transposed copies (an fp32 x holding the same bf16 values
    takes that path): same splits, same k order within each split."""
    rows, d_in, d_out = 16384, 1152, 3456
    announce(f"linear bwd token-major vs transposed rows={rows} d_out={d_out}")
    g = np.random.Generator(np.random.PCG64(790))
    x = round_bf16(g.standard_normal((rows, d_in)).astype(np.float32))
    w = round_bf16(g.standard_normal((d_out, d_in)).astype(np.float32) * 0.02)
    dy = round_bf16(g.standard_normal((rows, d_out)).astype(np.float32))
    _, dw_tn, db_tn = P.linear_bwd(dev(x, BF16), dev(w, BF16), dev(dy, BF16), want_dx=False)
    _, dw_t, db_t = P.linear_bwd(dev(x, F32), dev(w, BF16), dev(dy, BF16), want_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dw_tn, dw_t)
    np.testing.assert_allclose(host(db_tn), host(db_t), rtol=1e-5, atol=1e-4)


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
        assert_grad_close(dq[0, h], rq, f"dQ head {h}")
        assert_grad_close(dk[0, h], rk, f"dK head {h}")
        assert_grad_close(dv[0, h], rv, f"dV head {h}")


def test_attn_bwd_full_size_video_cross_attention(P):
    # cross-attention of the 16 x 30 x 45 video: 21600 token queries, 864
    # proxies (streamed query-major kernel), 16 heads; the oracle takes two
    # heads whole
    B, heads, Nq, Nk, dh = 1, 16, 21600, 864, 72
    announce("dense bwd full size video Nq=21600 Nk=864")
    q, k, v, do = make_attn_grad_inputs(B, heads, Nq, Nk, dh, seed=551)
    kv = dev(np.stack([k, v], axis=1), BF16)
    dq, dk, dv = P.attn_bwd(dev(q, BF16), kv[:, 0], kv[:, 1], dev(do, BF16))
    torch.cuda.synchronize()
    dq, dk, dv = host(dq), host(dk), host(dv)
    for h in (0, heads - 1):
        sl = slice(h * dh, (h + 1) * dh)
        rq, rk, rv = O.attention_bwd(q[0, h], k[0, h], v[0, h], do[0][:, sl], 1)
        assert_grad_close(dq[0, h], rq, f"dQ head {h}")
        assert_grad_close(dk[0, h], rk, f"dK head {h}")
        assert_grad_close(dv[0, h], rv, f"dV head {h}")


@pytest.mark.parametrize("d_in,d_out", [(1152, 1152), (1152, 3456), (64, 200)])
def test_linear_bwd_ex_joins(P, d_in, d_out):
    """ptdit_linear_bwd_ex against ptdit_linear_bwd: the bf16-only d_x is the
    nearest-even rounding of the fp32 d_x, bit for bit; d_x with an added
    gradient (out of place and in place) equals d_x + add to fp32 rounding
    (the K = 1152 products fold the addend into the accumulators mid-loop, so
    the order of the additions differs), and its bf16 copy rounds that sum."""
    from diffusion_transformer_attention_pt_amd import _lib
    from gpu_util import dev
    rows = 2400
    announce(f"linear_bwd_ex rows={rows} {d_in}->{d_out}")
    g = np.random.Generator(np.random.PCG64(700 + d_out))
    x = dev(round_bf16(g.standard_normal((rows, d_in)).astype(np.float32)), BF16)
    w = dev(round_bf16((g.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)), BF16)
    dy = dev(g.standard_normal((rows, d_out)).astype(np.float32), F32)
    add = dev(g.standard_normal((rows, d_in)).astype(np.float32), F32)
    dx0, dw0, db0 = _lib.linear_bwd(x, w, dy)
    b16 = torch.empty(rows, d_in, dtype=BF16, device="cuda")
    _, dw1, db1 = _lib.linear_bwd(x, w, dy, want_dx=False, dx_bf16=b16)
    torch.cuda.synchronize()
    assert torch.equal(b16.view(torch.int16), dx0.to(BF16).view(torch.int16))
    assert torch.equal(dw1, dw0) and torch.equal(db1, db0)
    ref = host(dx0).astype(np.float64) + host(add)
    tol = 1e-5 * max(1.0, float(np.abs(ref).max()))
    dx2 = torch.empty(rows, d_in, dtype=F32, device="cuda")
    b16b = torch.empty(rows, d_in, dtype=BF16, device="cuda")
    _lib.linear_bwd(x, w, dy, dx=dx2, dx_add=add, dx_bf16=b16b, want_dw=False, want_db=False)
    inplace = add.clone()
    _lib.linear_bwd(x, w, dy, dx=inplace, dx_add=inplace, want_dw=False, want_db=False)
    torch.cuda.synchronize()
    assert np.abs(host(dx2) - ref).max() <= tol
    assert np.abs(host(inplace) - ref).max() <= tol
    assert torch.equal(b16b.view(torch.int16), dx2.to(BF16).view(torch.int16))


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
    (130, 72, 200, "bf16", "bf16"),       # the weight's transposed copy ragged in both 64-wide tile axes
    (16384, 1152, 1152, "bf16", "f32"),   # the 2048^2 output projection
    # bf16 d_y and x, token counts a multiple of 128: dW from the token-major
    # operands directly (no transposed copies)
    (16384, 1152, 3456, "bf16", "bf16"),  # the 2048^2 Q/K/V projection: 4 splits of 4096
    (2432, 1152, 3456, "bf16", "bf16"),   # splits of 640 tokens, the last 512; 3456 rows of dW ragged in 256
    (1408, 1152, 1152, "bf16", "bf16"),   # a 128-token remainder joined to the last split (384)
    (256, 1152, 1152, "bf16", "bf16"),    # one split of 256 tokens
    # token counts a multiple of 32 only: the last split starts early and its
    # first slices read zeros
    (21600, 1152, 3456, "bf16", "bf16"),  # the 16 x 30 x 45 video's Q/K/V projection
    (1312, 1152, 1152, "bf16", "bf16"),   # splits of 256, the last 288 tokens in K 384: 3 zero slices
    (288, 1152, 1152, "bf16", "bf16"),    # one split, 288 tokens in K 384 (it starts 96 tokens early)
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
    # error 2^-9 per term); d_w and d_b sum `rows` terms of size ~1, so their
    # max-abs bar scales with their largest element (grad_bar)
    assert_grad_close(host(dx), rx, "dX")
    assert_grad_close(host(dw), rw, "dW")
    assert_grad_close(host(db), rb, "db")


@pytest.mark.parametrize("rows,d_in,d_out,n", [(16384, 1152, 1152, 4), (21600, 1152, 1152, 3),
                                               (4096, 1152, 3456, 2), (2400, 1152, 1152, 1)])
def test_linear_bwd_dw_group(P, rows, d_in, d_out, n):
    """ptdit_linear_bwd_dw_group: each product's dW against the float64
    oracle (gradient bar) and against its own ptdit_linear_bwd call (the same
    bf16 products summed in fp32 over other token splits: within fp32
    rounding); db bit for bit (the same column sums and split order)."""
    from diffusion_transformer_attention_pt_amd import _lib
    announce(f"grouped dW rows={rows} {d_in}->{d_out} n={n}")
    g = np.random.Generator(np.random.PCG64(900 + n + rows % 97))
    xs = [round_bf16(g.standard_normal((rows, d_in)).astype(np.float32)) for _ in range(n)]
    dys = [round_bf16(g.standard_normal((rows, d_out)).astype(np.float32)) for _ in range(n)]
    w = dev(round_bf16(g.standard_normal((d_out, d_in)).astype(np.float32) * 0.02), BF16)
    xd, dyd = [dev(a, BF16) for a in xs], [dev(a, BF16) for a in dys]
    dws, dbs = _lib.linear_bwd_dw_group(xd, dyd)
    torch.cuda.synchronize()
    for i in range(n):
        _, dw1, db1 = _lib.linear_bwd(xd[i], w, dyd[i], want_dx=False)
        torch.cuda.synchronize()
        got, one = host(dws[i]), host(dw1)
        assert np.abs(got - one).max() <= 2e-6 * max(1.0, float(np.abs(one).max())) * np.sqrt(rows), f"dW {i}"
        assert torch.equal(dbs[i], db1), f"db {i}"
    _, rw, rb = O.linear_bwd(xs[0], host(w), dys[0])
    assert_grad_close(host(dws[0]), rw, "grouped dW 0")
    assert_grad_close(host(dbs[0]), rb, "grouped db 0")


@pytest.mark.parametrize("rows,d_in,d_out,add", [(16384, 1152, 1152, True), (2400, 1152, 1152, True),
                                                 (4096, 1152, 1152, False), (1200, 1152, 1024, False),
                                                 (16384, 1152, 3456, True)])
def test_linear_bwd_dx_weight_as_it_lies(P, rows, d_in, d_out, add):
    """d_x = dY W from bf16 dY reads W [d_out][d_in] as it lies (the k-major
    instance of the ping-pong GEMM, no transposed copy): against the same
    product from an fp32 dY holding the same values (which takes the
    transposed copy) to fp32 summation order, with and without an added
    gradient (the residual in the main loop when d_out = 1152), ragged row
    tiles included; and against the float64 oracle."""
    from diffusion_transformer_attention_pt_amd import _lib
    announce(f"dX k-major W rows={rows} {d_out}->{d_in} add={add}")
    g = np.random.Generator(np.random.PCG64(960 + rows % 89 + d_out))
    x = round_bf16(g.standard_normal((rows, d_in)).astype(np.float32))
    w = round_bf16((g.standard_normal((d_out, d_in)) * 0.05).astype(np.float32))
    dy = round_bf16(g.standard_normal((rows, d_out)).astype(np.float32))
    ad = dev(g.standard_normal((rows, d_in)).astype(np.float32), F32) if add else None
    wd = dev(w, BF16)
    dx_k, _, _ = _lib.linear_bwd(dev(x, BF16), wd, dev(dy, BF16), want_dw=False, want_db=False,
                                 dx_add=ad, dx=torch.empty(rows, d_in, dtype=F32, device="cuda") if add else None)
    dx_t, _, _ = _lib.linear_bwd(dev(x, BF16), wd, dev(dy, F32), want_dw=False, want_db=False,
                                 dx_add=ad, dx=torch.empty(rows, d_in, dtype=F32, device="cuda") if add else None)
    torch.cuda.synchronize()
    k, t = host(dx_k), host(dx_t)
    assert np.abs(k - t).max() <= 1e-5 * max(1.0, float(np.abs(t).max())), "k-major vs transposed"
    ref = dy.astype(np.float64) @ w.astype(np.float64)
    if add:
        ref = ref + host(ad)
    assert_grad_close(k, ref, "dX k-major")
