"""GPU parity of the composed block backward (PTBlockBackward: the chain of
C-ABI calls) against the float64 block-backward oracle (oracle.block_bwd,
pinned to finite differences and torch autograd): the gradient of <x3, dout>
with respect to the block input and every weight and bias of the four
attentions, compared element by element.

Bar: reading R-gradbar (tests/gpu_util.py, grad_bar): relative-L2 1e-2 and
max-abs 2e-2 scaled by max(1, largest magnitude of the reference). The key biases are the
exception: a key bias adds q.b_k to every score of a query's row, which the
softmax cancels, so their exact gradient is zero and the oracle's value is
rounding noise; there the GPU value is held to the absolute bar scaled by the
value bias gradient of the same attention.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_grad_close, grad_bar, host
from synth_inputs import WORKLOADS, make_all_weights, make_x, tiny

pytestmark = pytest.mark.gpu

CASES = {
    # the 2048^2 block (64-token windows, 256 proxies)
    "img2048": WORKLOADS["img2048"],
    # a padded video grid: 30 x 45 pads to 32 x 48, 2 x 8 x 8 windows
    # (128 tokens) with the temporal shift, 216 proxies
    "video_pad": tiny("bwd_video", B=1, F=4, H=30, W=45, D=1152, heads=16, p=(1, 5, 5), win=(2, 8, 8),
                      shift=(1, 4, 4), dtype="bf16", index=61),
    # batch 2, 20 x 36 padded to 24 x 40 with a shift (2) that differs from the
    # pad (4): pad keys are visible, on the 64-token matrix-core kernels
    "batch2_pad": tiny("bwd_b2", B=2, F=1, H=20, W=36, D=1152, heads=16, p=(1, 4, 4), win=(1, 8, 8),
                       shift=(0, 2, 2), dtype="bf16", index=62),
    # half the 16 x 30 x 45 video: 432 proxies (more than 256 keys: the
    # streamed query-major kernels) and 2 x 8 x 8 windows (the 128-token
    # matrix-core window kernel), 30 x 45 padded to 32 x 48
    "video_432_proxies": tiny("bwd_video432", B=1, F=8, H=30, W=45, D=1152, heads=16, p=(1, 5, 5),
                              win=(2, 8, 8), shift=(1, 4, 4), dtype="bf16", index=64),
}


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_attention_pt_amd as P
    P.load()
    return P


@pytest.mark.parametrize("name", list(CASES))
def test_block_backward_vs_oracle(P, name):
    wl = CASES[name]
    announce(f"block backward {name} grid={(wl.B,) + wl.grid} p={wl.p} win={wl.win} shift={wl.shift}")
    x = make_x(wl)
    ws = make_all_weights(wl)
    g = np.random.Generator(np.random.PCG64(900 + wl.index))
    dout = g.standard_normal((wl.B, wl.N, wl.D)).astype(np.float32)
    blk = P.PTBlockAttention(wl.B, wl.grid, wl.D, wl.heads, wl.p, wl.win, wl.shift, ws, prec=torch.bfloat16)
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    bwd = P.PTBlockBackward(blk)
    ref = O.block_bwd(x, wl.grid, wl.p, wl.win, wl.shift, ws, wl.heads, dout, pool="f32")
    # recompute mode (forward for inference), then keep mode (the forward's
    # Q/K/V and attention outputs read back instead of recomputed)
    for keep in (False, True):
        announce(f"  keep={keep}")
        blk.forward(xd, keep=keep)
        got = bwd.backward(xd, torch.from_numpy(dout).cuda())
        torch.cuda.synchronize()
        _check_block_grads(got, ref, wl.D)


def _check_block_grads(got, ref, D):
    assert_grad_close(host(got["dx"]), ref["dx"], "dx")
    for a, att in enumerate(("proxy SA", "cross", "WSA", "SWSA")):
        gw, rw = got["weights"][a], ref["weights"][a]
        wqkv, bqkv = host(gw["w_qkv"]), host(gw["b_qkv"])
        for i, n in enumerate("qkv"):
            assert_grad_close(wqkv[i * D:(i + 1) * D], rw["w" + n], f"{att} dW{n}")
        assert_grad_close(bqkv[:D], rw["bq"], f"{att} db_q")
        assert_grad_close(bqkv[2 * D:], rw["bv"], f"{att} db_v")
        # key bias: exactly zero in exact arithmetic (softmax shift invariance)
        assert np.abs(rw["bk"]).max() < 1e-9
        bar = grad_bar(rw["bv"])
        mk = float(np.abs(bqkv[D:2 * D]).max())
        print(f"  {att} db_k: max-abs {mk:.3e} (bar {bar:.3e}, exact value 0)", flush=True)
        assert mk <= bar
        assert_grad_close(host(gw["w_o"]), rw["wo"], f"{att} dW_o")
        assert_grad_close(host(gw["b_o"]), rw["bo"], f"{att} db_o")


@pytest.mark.parametrize("name", ["batch2_pad", "img2048"])
def test_grouped_weight_gradients_match_the_chain(P, name):
    """PTBlockBackward with the four D x D weight gradients grouped at the end
    (ptdit_linear_bwd_dw_group, the default) against the chain that forms
    them in place: d_x and every other gradient bit for bit (the same calls),
    the grouped d_W within fp32 rounding of the chain's (the same bf16
    products summed over other token splits), their d_b bit for bit."""
    wl = CASES[name]
    announce(f"grouped vs in-chain weight gradients {name}")
    x = make_x(wl)
    ws = make_all_weights(wl)
    g = np.random.Generator(np.random.PCG64(950 + wl.index))
    dout = torch.from_numpy(g.standard_normal((wl.B, wl.N, wl.D)).astype(np.float32)).cuda()
    blk = P.PTBlockAttention(wl.B, wl.grid, wl.D, wl.heads, wl.p, wl.win, wl.shift, ws, prec=torch.bfloat16)
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    b_grp, b_chain = P.PTBlockBackward(blk), P.PTBlockBackward(blk, group_dw=False)
    assert b_grp.group and not b_chain.group
    for keep in (False, True):
        blk.forward(xd, keep=keep)
        a = b_grp.backward(xd, dout)
        a = {"dx": a["dx"].clone(), "weights": [{k: v.clone() for k, v in w.items()} for w in a["weights"]]}
        c = b_chain.backward(xd, dout)
        torch.cuda.synchronize()
        assert torch.equal(a["dx"], c["dx"]), "dx"
        D = wl.D
        grouped = {(1, "w_o"), (2, "w_o"), (3, "w_o")}
        for i in range(4):
            for k in ("w_qkv", "b_qkv", "w_o", "b_o"):
                ga, gc = a["weights"][i][k], c["weights"][i][k]
                if (i, k) in grouped or (i == 1 and k == "w_qkv"):
                    rows = slice(0, D) if k == "w_qkv" else slice(None)
                    if k == "w_qkv":   # only the query rows are grouped
                        assert torch.equal(ga[D:], gc[D:]), f"{i} {k} K/V rows"
                    da, dc = host(ga[rows]), host(gc[rows])
                    assert np.abs(da - dc).max() <= 1e-5 * max(1.0, float(np.abs(dc).max())), f"{i} {k}"
                elif k == "b_qkv" and i >= 2:
                    # the window attentions' pad-slot key/value bias gradients
                    # are added with atomics (order of arrival): K/V rows close
                    assert torch.equal(ga[:D], gc[:D]), f"{i} {k} Q rows"
                    da, dc = host(ga[D:]), host(gc[D:])
                    assert np.abs(da - dc).max() <= 1e-5 * max(1.0, float(np.abs(dc).max())), f"{i} {k} K/V rows"
                else:
                    assert torch.equal(ga, gc), f"{i} {k}"


@pytest.mark.parametrize("name,prec", [("batch2_pad", torch.bfloat16), ("video_pad", torch.bfloat16),
                                       ("batch2_pad", torch.float32)])
def test_keep_mode_tensors(P, name, prec):
    """What a keep-mode forward leaves for the backward: the block output is
    bit for bit the recompute-mode output (the same kernels; keep only adds
    writes); the proxy SA and cross-attention Q/K/V and outputs are bit for
    bit what the backward's recompute calls produce (the same projection and
    attention kernels); so are the window attentions' Q/K/V and outputs,
    which with bf16 come from the fused projection + attention kernel: it
    takes the projection's k order, roundings and attention steps of the
    separate calls."""
    from diffusion_transformer_attention_pt_amd import _lib
    wl = CASES[name]
    announce(f"keep tensors {name} {prec} grid={(wl.B,) + wl.grid} win={wl.win} shift={wl.shift}")
    B, N, M, D, heads = wl.B, wl.N, wl.M, wl.D, wl.heads
    x = make_x(wl)
    blk = P.PTBlockAttention(wl.B, wl.grid, wl.D, wl.heads, wl.p, wl.win, wl.shift, make_all_weights(wl),
                             prec=prec)
    xd = torch.from_numpy(x).to(prec).cuda()
    y0 = blk.forward(xd).clone()
    y1 = blk.forward(xd, keep=True)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "keep changed the block output"
    k = blk.kept
    w = blk.weights
    xl = lambda t, lo: (lo if lo is not None else t.to(prec))
    # proxy SA: Q/K/V of P, attention of them
    qkvp = _lib.linear_heads(blk.P.view(B * M, D), w[0].w_qkv, w[0].b_qkv, B, M, heads)
    op = _lib.attn(qkvp[:, 0], qkvp[:, 1], qkvp[:, 2])
    torch.cuda.synchronize()
    assert torch.equal(k["sa_qkv"], qkvp), "proxy SA Q/K/V"
    assert torch.equal(k["sa_o"], op), "proxy SA output"
    # cross-attention: Q of the tokens, K/V of P'
    wc = w[1]
    q = _lib.linear_heads(xd.view(B * N, D), wc.w_qkv[:D], wc.b_qkv[:D], B, N, heads)
    kv = _lib.linear_heads(blk.P2.view(B * M, D), wc.w_qkv[D:], wc.b_qkv[D:], B, M, heads)
    o = _lib.attn(q[:, 0], kv[:, 0], kv[:, 1])
    torch.cuda.synchronize()
    assert torch.equal(k["x_q"], q), "cross-attention Q"
    assert torch.equal(k["x_kv"], kv), "cross-attention K/V"
    assert torch.equal(k["x_o"], o), "cross-attention output"
    # window attentions
    for nm, src, lo, wt, sh in (("wsa", blk.x1, blk.x1_lowp, w[2], (0, 0, 0)),
                                ("swsa", blk.x2, blk.x2_lowp, w[3], wl.shift)):
        a = xl(src, lo).view(B * N, D)
        qkv = _lib.linear_heads(a, wt.w_qkv, wt.b_qkv, B, N, heads)
        ow = _lib.window_attn(qkv, wt.b_qkv, blk.g, wl.win, sh)
        torch.cuda.synchronize()
        assert torch.equal(k[nm + "_qkv"], qkv), nm + " Q/K/V"
        assert torch.equal(k[nm + "_o"], ow), nm + " output"


def test_chaining_primitives(P):
    """The recompute and chaining calls on their own: the head-major
    projection and the two attention cores against the oracle's linear map,
    window core and attention (bar as everywhere); the layout change, the
    bf16 rounding (round to nearest even, as torch casts) and the fp32 add
    bit for bit."""
    from diffusion_transformer_attention_pt_amd import _lib
    from gpu_util import assert_close, dev
    wl = tiny("prims", B=2, F=1, H=20, W=36, D=1152, heads=16, p=(1, 4, 4), win=(1, 8, 8), shift=(0, 2, 2),
              dtype="bf16", index=63)
    B, N, D, heads = wl.B, wl.N, wl.D, wl.heads
    dh = D // heads
    x = make_x(wl)
    w = make_all_weights(wl)[3]
    aw = P.AttnWeights.from_dict(w, torch.bfloat16, "cuda")
    qkv = _lib.linear_heads(dev(x, torch.bfloat16).view(B * N, D), aw.w_qkv, aw.b_qkv, B, N, heads)
    torch.cuda.synchronize()
    toks = lambda t: t.transpose(0, 2, 1, 3).reshape(B, -1, D)       # [B, heads, L, dh] -> [B, L, D]
    q64 = [O.linear(x, w["w" + n], w["b" + n]) for n in "qkv"]
    for i, n in enumerate("qkv"):
        assert_close(toks(host(qkv[:, i])), q64[i], f"linear_heads {n}")
    o = _lib.window_attn(qkv, aw.b_qkv, (B, 1, wl.H, wl.W, D, heads), wl.win, wl.shift)
    q16 = [toks(host(qkv[:, i])) for i in range(3)]   # the bf16 Q/K/V the core reads
    ref = O.window_core(q16[0], q16[1], q16[2], wl.grid, wl.win, wl.shift, heads, host(aw.b_qkv)[D:2 * D],
                        host(aw.b_qkv)[2 * D:])
    assert_close(host(o), ref, "window_attn")
    M = 250
    kv = qkv[:, 1:, :, :M].contiguous()
    oa = _lib.attn(qkv[:, 0], kv[:, 0], kv[:, 1])
    ref = O.attention(q16[0], toks(host(kv[:, 0])), toks(host(kv[:, 1])), heads)
    assert_close(host(oa), ref, "attn")
    g = np.random.Generator(np.random.PCG64(64))
    src = g.standard_normal((B, 3, heads, N, dh)).astype(np.float32)
    t = _lib.heads_to_tokens(dev(src, torch.float32))
    np.testing.assert_array_equal(host(t), src.transpose(0, 3, 1, 2, 4).reshape(B, N, 3 * D))
    a = dev(g.standard_normal((B, N, D)).astype(np.float32) * 7, torch.float32)
    b = dev(g.standard_normal((B, N, D)).astype(np.float32), torch.float32)
    assert torch.equal(_lib.f32_to_bf16(a).view(torch.int16), a.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(_lib.add_f32(a, b), a + b)
    c = a.clone()
    _lib.add_f32(c, b, out=c)                    # in place
    assert torch.equal(c, a + b)
