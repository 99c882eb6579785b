"""Backward of the PT-block attention core as a chain of C-ABI calls.

The gradient of <x3, dout> with respect to the block input x and the 32
weight and bias tensors of its four attentions (Qihoo-T2X reading note,
section 3, Eq. GIIM and Eq. TCM, in the order of the code-correspondence
excerpt of the PT-Block forward; the pages train at 2048^2, section 4). The
calls run in reverse order of the forward:

    x3 = x2 + SWSA(x2)   ->  dx2 = dout + dSWSA/dx2^T dout
    x2 = x1 + WSA(x1)    ->  dx1 = dx2 + dWSA/dx1^T dx2
    x1 = x + CS(x, P')   ->  dx  = dx1 + dCS/dx^T dx1,   dP' = dCS/dP'^T dx1
    P' = P + SA(P)       ->  dP  = dP' + dSA/dP^T dP'
    P  = Averaging(x)    ->  dx += Averaging^T dP

Each attention's backward takes its head-major Q/K/V and attention output
from the forward when it ran with keep=True (the calls' workspaces, kept
apart), else recomputes them (ptdit_linear_heads, ptdit_window_attn /
ptdit_attn) from the block's stored inputs. Then come the output projection's
gradient (ptdit_linear_bwd_ex, whose d_x product writes the core's bf16 dO
directly), the core's (ptdit_window_attn_bwd_tokens / ptdit_attn_bwd) and the
input projections' (ptdit_linear_bwd_ex on the token-major dQ/dK/dV: the
window cores write them so, in bf16, the precision the projection's gradient
products read them in; the cross-attention core writes its dQ so too,
ptdit_attn_bwd_tokens; the proxy keys' and values' gradients pass through
ptdit_heads_to_tokens), the residual branch's gradient added in the d_x
product's epilogue. The output projections' gradient products read bf16 dY
(the precision their operands take anyway): dout rounded by
ptdit_f32_to_bf16, dx2 and dx1 written in bf16 beside fp32 by the products
that form them; with bf16 operands and a token count that is a multiple of
128 the weight gradients need no transposed copies. The window average's
gradient accumulates into dx (ptdit_proxy_pool_bwd). Every step runs in the
library's kernels; torch only holds the buffers. bf16 precision blocks with
window-average proxies.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from . import _lib
from .block import PTBlockAttention


class PTBlockBackward:
    def __init__(self, blk: PTBlockAttention, group_dw: bool = True):
        """group_dw: leave the weight and bias gradients of the four N-row
        D x D maps (the three output projections of the token rows and the
        cross-attention's query projection) to the end of the pass, where one
        ptdit_linear_bwd_dw_group launch forms all four (fewer token splits
        and partial sums than four calls); the chain then forms only their
        d_x products. Where that call's shape rules do not hold (fewer than
        256 or a count of tokens not a multiple of 32, D < 1024) the
        gradients stay in the chain."""
        if blk.prec != torch.bfloat16:
            raise ValueError("the block backward runs on bf16 blocks (bf16 matrix-core gradient kernels)")
        if blk.proxy_mode != "mean" or blk.full:
            raise ValueError("the block backward covers the attention core with window-average proxies")
        self.blk = blk
        B, N, M, D, heads = blk.B, blk.N, blk.M, blk.D, blk.heads
        dh = D // heads
        dev = blk.device
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=f32: torch.empty(*s, dtype=dt, device=dev)
        self.pads = any(g % w for g, w in zip((blk.F, blk.H, blk.W), blk.win))
        # token-row buffers (shared by both window attentions)
        self.qkv = e(B, 3, heads, N, dh, dt=bf)
        self.o = e(B, N, D, dt=bf)
        self.do16 = e(B, N, D, dt=bf)
        self.dqkv_t16 = e(B, N, 3 * D, dt=bf)   # the window cores' gradient, token-major bf16
        self.dbkv = e(2, D)
        self.dx2, self.dx1, self.dx = e(B, N, D), e(B, N, D), e(B, N, D)
        # bf16 copies of the residual-stream gradients for the output
        # projections' gradient products (dout's, then dx1's; dx2's)
        self.g16a, self.g16b = e(B, N, D, dt=bf), e(B, N, D, dt=bf)
        # cross-attention and proxy buffers
        self.q = e(B, 1, heads, N, dh, dt=bf)
        self.kv = e(B, 2, heads, M, dh, dt=bf)
        self.dkv_h = e(B, 2, heads, M, dh)
        self.dkv_t = e(B, M, 2 * D)
        self.qkvp = e(B, 3, heads, M, dh, dt=bf)
        self.op = e(B, M, D, dt=bf)
        self.dop16 = e(B, M, D, dt=bf)
        self.dqkvp_h = e(B, 3, heads, M, dh)
        self.dqkvp_t = e(B, M, 3 * D)
        self.dP = e(B, M, D)
        lib = _lib.load()
        gneed = int(lib.ptdit_linear_bwd_dw_group_workspace_bytes(4, B * N, D, D))
        self.group = group_dw and gneed > 0
        if self.group:
            # operands kept for the deferred products: bf16(dout) (g16a is
            # reused for dx1), and the recompute path's attention outputs
            self.g16c = e(B, N, D, dt=bf)
            self.o_w2, self.o_x = e(B, N, D, dt=bf), e(B, N, D, dt=bf)
        need = max(gneed, int(lib.ptdit_linear_bwd_workspace_bytes(B * N, D, 3 * D)),
                   int(lib.ptdit_linear_bwd_workspace_bytes(B * M, D, 3 * D)),
                   int(lib.ptdit_attn_bwd_workspace_bytes(B, heads, N, M, dh)),
                   int(lib.ptdit_attn_bwd_workspace_bytes(B, heads, M, M, dh)))
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def _window(self, xl: torch.Tensor, w: _lib.AttnWeights, shift, dy: torch.Tensor, dx_out: torch.Tensor,
                kept=None, dy16=None, dx_out16=None, o_buf=None):
        """One window attention's backward: returns its weight gradients and
        writes dx_out = dy + d(branch)/dx^T dy (and its bf16 copy into
        dx_out16). kept: (qkv, o) of the forward; dy16: bf16(dy), which the
        output projection's gradient products read."""
        blk = self.blk
        B, N, D, heads = blk.B, blk.N, blk.D, blk.heads
        if kept is not None:
            qkv, o = kept
        else:
            qkv, o = self.qkv, (o_buf if o_buf is not None else self.o)
            _lib.linear_heads(xl.view(B * N, D), w.w_qkv, w.b_qkv, B, N, heads, out=qkv)
            _lib.window_attn(qkv, w.b_qkv, blk.g, blk.win, shift, out=o)
        dyo = dy16 if dy16 is not None else dy
        if self.group:   # dW, db of w_o at the end of the pass
            _lib.linear_bwd(o, w.w_o, dyo, ws=self.ws, want_dx=False, want_dw=False, want_db=False,
                            dx_bf16=self.do16)
            dwo = torch.empty(D, D, dtype=torch.float32, device=o.device)
            dbo = torch.empty(D, dtype=torch.float32, device=o.device)
            self._deferred.append((o, dyo, dwo, dbo))
        else:
            _, dwo, dbo = _lib.linear_bwd(o, w.w_o, dyo, ws=self.ws, want_dx=False, dx_bf16=self.do16)
        if self.pads:
            self.dbkv.zero_()
        # dQ/dK/dV written token-major: the Q/K/V projection's d_y as it is read
        _lib.window_attn_bwd(qkv, self.do16, blk.g, blk.win, shift, b_qkv=w.b_qkv, d_qkv=self.dqkv_t16,
                             d_b_kv=self.dbkv if self.pads else None, tokens=True, pad_grad=self.pads)
        # dx_out = dy (the residual) + d(branch)/dx^T dy, joined in the product
        _, dwqkv, dbqkv = _lib.linear_bwd(xl, w.w_qkv, self.dqkv_t16, ws=self.ws, dx=dx_out, dx_add=dy,
                                          dx_bf16=dx_out16)
        if self.pads:   # pad slots' key/value gradients reach b_k, b_v
            _lib.add_f32(dbqkv[D:], self.dbkv.view(-1), out=dbqkv[D:])
        return {"w_qkv": dwqkv, "b_qkv": dbqkv, "w_o": dwo, "b_o": dbo}

    def backward(self, x: torch.Tensor, dout: torch.Tensor) -> Dict[str, object]:
        """Gradients after blk.forward(x) or blk.forward(x, keep=True) (whose
        intermediates it reads; with keep, also its Q/K/V and attention outputs).
        dout: fp32 [B, N, D]. Returns {"dx": fp32 [B, N, D], "weights": [per
        attention (proxy SA, cross, WSA, SWSA) {"w_qkv", "b_qkv", "w_o",
        "b_o"}]} (all fp32)."""
        blk = self.blk
        B, N, M, D, heads = blk.B, blk.N, blk.M, blk.D, blk.heads
        w = blk.weights
        if dout.dtype != torch.float32 or not dout.is_contiguous():
            raise ValueError("dout must be a contiguous fp32 tensor")
        grads: List[dict] = [None] * 4
        k = blk.kept
        self._deferred = []   # (X, dY, dW, db) of the grouped D x D products
        # the output projections' gradient products take bf16(dY): dout's
        # rounded here, dx2's and dx1's written by the products that form them
        dout16 = self.g16c if self.group else self.g16a
        _lib.f32_to_bf16(dout, out=dout16)
        grads[3] = self._window(blk.x2_lowp, w[3], blk.shift, dout, self.dx2,
                                kept=(k["swsa_qkv"], k["swsa_o"]) if k else None, dy16=dout16,
                                dx_out16=self.g16b)
        grads[2] = self._window(blk.x1_lowp, w[2], (0, 0, 0), self.dx2, self.dx1,
                                kept=(k["wsa_qkv"], k["wsa_o"]) if k else None, dy16=self.g16b,
                                dx_out16=self.g16a, o_buf=self.o_w2 if self.group else None)
        # cross-attention: tokens are queries, the attended proxies P' keys/values
        wc = w[1]
        if k:
            q, kv, o = k["x_q"], k["x_kv"], k["x_o"]
        else:
            q, kv, o = self.q, self.kv, (self.o_x if self.group else self.o)
            _lib.linear_heads(x.view(B * N, D), wc.w_qkv[:D], wc.b_qkv[:D] if wc.b_qkv is not None else None,
                              B, N, heads, out=q)
            _lib.linear_heads(blk.P2.view(B * M, D), wc.w_qkv[D:], wc.b_qkv[D:] if wc.b_qkv is not None else None,
                              B, M, heads, out=kv)
            _lib.attn(q[:, 0], kv[:, 0], kv[:, 1], out=o)
        if self.group:
            _lib.linear_bwd(o, wc.w_o, self.g16a, ws=self.ws, want_dx=False, want_dw=False, want_db=False,
                            dx_bf16=self.do16)
            dwo = torch.empty(D, D, dtype=torch.float32, device=x.device)
            dbo = torch.empty(D, dtype=torch.float32, device=x.device)
            self._deferred.append((o, self.g16a, dwo, dbo))
        else:
            _, dwo, dbo = _lib.linear_bwd(o, wc.w_o, self.g16a, ws=self.ws, want_dx=False, dx_bf16=self.do16)
        # dQ token-major bf16 [B, N, D] into the (now free) window gradient buffer
        dq_t = self.dqkv_t16.view(-1)[:B * N * D].view(B, N, D)
        _lib.attn_bwd(q[:, 0], kv[:, 0], kv[:, 1], self.do16, ws=self.ws,
                      dq=dq_t, dk=self.dkv_h[:, 0], dv=self.dkv_h[:, 1], dq_tokens=True)
        dwqkv = torch.empty(3 * D, D, dtype=torch.float32, device=x.device)
        dbqkv = torch.empty(3 * D, dtype=torch.float32, device=x.device)
        # dx = dx1 (the residual) + the queries' gradient, joined in the product
        if self.group:
            _lib.linear_bwd(x, wc.w_qkv[:D], dq_t, ws=self.ws, dx=self.dx, dx_add=self.dx1, want_dw=False,
                            want_db=False)
            self._deferred.append((x, dq_t, dwqkv[:D], dbqkv[:D]))
        else:
            _lib.linear_bwd(x, wc.w_qkv[:D], dq_t, ws=self.ws, dx=self.dx, dx_add=self.dx1, dw=dwqkv[:D],
                            db=dbqkv[:D])
        _lib.heads_to_tokens(self.dkv_h, out=self.dkv_t)
        dP2, _, _ = _lib.linear_bwd(blk.P2, wc.w_qkv[D:], self.dkv_t, ws=self.ws, dw=dwqkv[D:], db=dbqkv[D:])
        grads[1] = {"w_qkv": dwqkv, "b_qkv": dbqkv, "w_o": dwo, "b_o": dbo}
        # proxy self-attention on P (queries = keys = proxies)
        wp = w[0]
        if k:
            qkvp, op = k["sa_qkv"], k["sa_o"]
        else:
            qkvp, op = self.qkvp, self.op
            _lib.linear_heads(blk.P.view(B * M, D), wp.w_qkv, wp.b_qkv, B, M, heads, out=qkvp)
            _lib.attn(qkvp[:, 0], qkvp[:, 1], qkvp[:, 2], out=op)
        _, dwo0, dbo0 = _lib.linear_bwd(op, wp.w_o, dP2, ws=self.ws, want_dx=False, dx_bf16=self.dop16)
        _lib.attn_bwd(qkvp[:, 0], qkvp[:, 1], qkvp[:, 2], self.dop16, ws=self.ws,
                      dq=self.dqkvp_h[:, 0], dk=self.dqkvp_h[:, 1], dv=self.dqkvp_h[:, 2])
        _lib.heads_to_tokens(self.dqkvp_h, out=self.dqkvp_t)
        # dP = dP' (the residual) + the proxy attention's gradient
        _, dwqkv0, dbqkv0 = _lib.linear_bwd(blk.P, wp.w_qkv, self.dqkvp_t, ws=self.ws, dx=self.dP, dx_add=dP2)
        grads[0] = {"w_qkv": dwqkv0, "b_qkv": dbqkv0, "w_o": dwo0, "b_o": dbo0}
        # window average: every token of a window receives dP / P
        _lib.proxy_pool_bwd(self.dP, blk.g, blk.p, d_x=self.dx, accumulate=True)
        if self._deferred:   # the four D x D maps' dW, db in one launch
            xs, dys, dws, dbs = (list(t) for t in zip(*self._deferred))
            _lib.linear_bwd_dw_group([a.reshape(B * N, D) for a in xs], [a.reshape(B * N, D) for a in dys], dws,
                                     dbs, ws=self.ws)
            self._deferred = []
        return {"dx": self.dx, "weights": grads}
