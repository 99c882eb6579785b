"""GPU parity of the fused Q/K/V projection + window attention kernel
(csrc/wfused.hip), the path ptdit_window_sa / ptdit_shift_window_sa take for
bf16 operands with head width 72 and windows of 32, 64 or 128 tokens.

Each case checks, through the C ABI:
  * that the fused kernel ran (the library's kernel trace of its class);
  * the branch output (residual off) and the call with the residual against
    the float64 oracle (max-abs 2e-2, relative-L2 1e-2);
  * equality, bit for bit, with the unfused path (projection GEMM to a
    head-major Q/K/V workspace, then the window kernel), which an fp32 input
    without a bf16 copy takes: both compute the same bf16 Q/K/V in the same
    order and the same attention steps;
  * the keep variant (ptdit_window_sa_keep): the same output, and the Q/K/V
    it copies out equal, bit for bit, to the unfused path's.
Cases span padded grids, shifts that differ from the pad, 3D 128-token
windows, 32-token windows, row tiles that straddle a batch boundary, a head
count other than 16, the full 2048^2 grid, and the shapes the fused kernel
leaves to the unfused path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_close, dev, host
from synth_inputs import make_weights, make_x, tiny

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_attention_pt_amd as P
    P.load()
    return P


def _wl(**kw):
    base = dict(B=1, F=1, H=24, W=40, D=1152, heads=16, p=(1, 4, 4), win=(1, 8, 8), shift=(0, 4, 4),
                dtype="bf16", index=31)
    base.update(kw)
    return tiny("wfused", **base)


CASES = {
    "img_shift": _wl(),
    "img_noshift": _wl(shift=(0, 0, 0)),
    # 20 x 36 pads to 24 x 40 (pad 4) with a shift of 2: pad keys are seen
    "pad_shift2": _wl(H=20, W=36, shift=(0, 2, 2)),
    # 2 x 8 x 8 windows (128 tokens), padded in every axis, temporal shift
    "video_pad": _wl(F=3, H=10, W=12, win=(2, 8, 8), shift=(1, 4, 4)),
    "video_dma": _wl(F=3, H=30, W=45, win=(2, 8, 8), shift=(1, 4, 4)),
    # 32-token windows (two pairs a ring slot)
    "win32": _wl(H=16, W=40, win=(1, 4, 8), shift=(0, 2, 4)),
    # 960 slots a batch item: 128-slot tiles straddle the batch boundary
    "batch2_straddle": _wl(B=2, H=20, W=36, shift=(0, 4, 2)),
    # 32 heads of 72 (D = 2304): sixteen head pairs, so the XCD order gives
    # each XCD two pairs
    "heads32": _wl(D=2304, heads=32, H=16, W=24),
    # the 2048^2 grid with the TCM shift
    "img2048": _wl(H=128, W=128, p=(1, 8, 8)),
}


def _fused_launches(P, fn):
    from diffusion_transformer_attention_pt_amd import _lib
    _lib.trace_enable(_lib.K_WINDOW_FUSED, 16)
    try:
        out = fn()
        torch.cuda.synchronize()
        n = len(_lib.trace_read(16))
    finally:
        _lib.trace_disable()
    return out, n


@pytest.mark.parametrize("name", list(CASES))
def test_fused_window_calls(P, name):
    from diffusion_transformer_attention_pt_amd import _lib
    wl = CASES[name]
    g = (wl.B, wl.F, wl.H, wl.W, wl.D, wl.heads)
    announce(f"fused window {name} grid={(wl.B,) + wl.grid} D={wl.D} heads={wl.heads} win={wl.win} "
             f"shift={wl.shift}")
    x = make_x(wl, seed=800 + wl.index)
    for a, shifted in ((2, False), (3, True)):
        w = make_weights(wl, a)
        aw = P.AttnWeights.from_dict(w, BF16, "cuda")
        sh = wl.shift if shifted else (0, 0, 0)

        def call(xin, residual, x_lowp=None):
            if shifted:
                return P.shift_window_sa(xin, g, wl.win, sh, aw, residual=residual, out_dtype=F32, x_lowp=x_lowp)
            return P.window_sa(xin, g, wl.win, aw, residual=residual, out_dtype=F32, x_lowp=x_lowp)

        xb = dev(x, BF16)
        got, n = _fused_launches(P, lambda: call(xb, False))
        assert n == 1, f"fused kernel launches: {n}"
        ref = O.shift_window_sa(x, wl.grid, wl.win, sh, w, wl.heads, False)
        assert_close(host(got), ref, f"{'swsa' if shifted else 'wsa'} branch")
        # with w_qkv packed once by ptdit_pack_window_weights (no per-call
        # packing): the same bits
        aw_p = P.AttnWeights(aw.w_qkv, aw.b_qkv, aw.w_o, aw.b_o, _lib.pack_window_weights(aw, wl.heads))
        assert aw_p.w_qkv_packed is not None
        got_p, n_p = _fused_launches(P, lambda: (P.shift_window_sa(xb, g, wl.win, sh, aw_p, residual=False,
                                                                   out_dtype=F32) if shifted else
                                                 P.window_sa(xb, g, wl.win, aw_p, residual=False, out_dtype=F32)))
        assert n_p == 1
        assert torch.equal(got_p, got), "prepacked weights changed the output"
        # the unfused path (fp32 input, no bf16 copy) gives the same bits
        x32 = dev(x, F32)
        plain, n0 = _fused_launches(P, lambda: call(x32, False))
        assert n0 == 0
        assert torch.equal(got, plain), "fused and unfused paths differ"
        # with the residual: fp32 input plus its bf16 copy (the block's call)
        res, n1 = _fused_launches(P, lambda: call(x32, True, x_lowp=xb))
        assert n1 == 1
        assert_close(host(res), O.shift_window_sa(x, wl.grid, wl.win, sh, w, wl.heads, True),
                     f"{'swsa' if shifted else 'wsa'} + residual")
        # keep mode (ptdit_window_sa_keep): the same output, and the head-major
        # Q/K/V and attention output it leaves in the workspace equal, bit for
        # bit, what the unfused path leaves there (its projection GEMM's Q/K/V)
        need = _lib.workspace_bytes(_lib.OP_WINDOW_SA, g, 0, wl.win, BF16)
        ws_f = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")
        ws_u = torch.zeros(need, dtype=torch.uint8, device="cuda")
        kept, nk = _fused_launches(P, lambda: _lib.window_sa_keep(xb, g, wl.win, sh, aw, ws_f, residual=False,
                                                                  out_dtype=F32))
        assert nk == 1
        assert torch.equal(kept, got), "keep changed the output"
        _lib.window_sa_keep(x32, g, wl.win, sh, aw, ws_u, residual=False, out_dtype=F32)
        torch.cuda.synchronize()
        (qf, of), (qu, ou) = _lib.window_ws_views(ws_f, g, BF16), _lib.window_ws_views(ws_u, g, BF16)
        assert torch.equal(qf.view(torch.int16), qu.view(torch.int16)), "kept Q/K/V differ from the unfused path's"
        assert torch.equal(of.view(torch.int16), ou.view(torch.int16)), "kept outputs differ"


def test_fused_not_taken_where_unsupported(P):
    """Windows of other sizes, head width 64 and a width that is not a
    multiple of 128 (8 heads of 72) keep the unfused path."""
    for kw in (dict(win=(1, 4, 4), shift=(0, 2, 2)), dict(D=1024, heads=16, H=16, W=16),
               dict(D=576, heads=8, H=16, W=24)):
        wl = _wl(**kw)
        g = (wl.B, wl.F, wl.H, wl.W, wl.D, wl.heads)
        x = make_x(wl, seed=850)
        w = make_weights(wl, 3)
        aw = P.AttnWeights.from_dict(w, BF16, "cuda")
        got, n = _fused_launches(P, lambda: P.shift_window_sa(dev(x, BF16), g, wl.win, wl.shift, aw,
                                                              residual=False, out_dtype=F32))
        assert n == 0
        assert_close(host(got), O.shift_window_sa(x, wl.grid, wl.win, wl.shift, w, wl.heads, False),
                     f"unfused {kw}")


def test_packed_window_weights_layout(P):
    """ptdit_pack_window_weights is a pure permutation of w_qkv, pinned here
    by rebuilding it on the host: for head pair hp and k-slice kt, tile row r
    (V's 144 rows of the pair, then Q's, then K's) and 16-byte position q,
    the chunk (q ^ ((r >> 1) & 3)) of that weight row's k-slice."""
    from diffusion_transformer_attention_pt_amd import _lib
    for D, heads in ((1152, 16), (2304, 32)):
        announce(f"packed window weights D={D} heads={heads}")
        g = torch.Generator().manual_seed(D)
        w = (torch.randn(3 * D, D, generator=g) * 0.02).to(BF16)
        aw = P.AttnWeights(w.cuda(), None, torch.zeros(D, D, dtype=BF16, device="cuda"), None)
        got = _lib.pack_window_weights(aw, heads)
        torch.cuda.synchronize()
        hp_n, kt_n = heads // 2, D // 32
        hp = np.arange(hp_n)[:, None, None, None, None]
        kt = np.arange(kt_n)[None, :, None, None, None]
        r = np.arange(432)[None, None, :, None, None]
        q = np.arange(4)[None, None, None, :, None]
        e = np.arange(8)[None, None, None, None, :]
        tg, cc = r // 144, r % 144
        wrow = np.where(tg == 0, 2, tg - 1) * D + hp * 144 + cc
        col = kt * 32 + (q ^ ((r >> 1) & 3)) * 8 + e
        ref = w.view(torch.int16).numpy()[wrow, col]
        assert np.array_equal(got.view(torch.int16).cpu().numpy().reshape(ref.shape), ref)


def test_block_repacks_changed_window_weights(P):
    """PTBlockAttention reads its window attentions' packed w_qkv: after an
    in-place change of the weights, repack_weights() makes the forward follow
    it (equal, bit for bit, to a block built on the changed weights)."""
    wl = _wl(H=16, W=24)
    announce("block repack after an in-place weight change")
    from synth_inputs import make_all_weights
    ws = make_all_weights(wl)
    x = dev(make_x(wl, seed=870), BF16)
    blk = P.PTBlockAttention(wl.B, wl.grid, wl.D, wl.heads, wl.p, wl.win, wl.shift, ws, prec=BF16)
    ws2 = [dict(w) for w in ws]
    ws2[3] = dict(ws[3], wq=ws[3]["wq"] * 1.5)
    ref = P.PTBlockAttention(wl.B, wl.grid, wl.D, wl.heads, wl.p, wl.win, wl.shift, ws2, prec=BF16).forward(x).clone()
    D = wl.D
    blk.weights[3].w_qkv[:D].copy_(torch.as_tensor(ws2[3]["wq"]).to(BF16))
    blk.repack_weights()
    got = blk.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
