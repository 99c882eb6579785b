"""The attention core of one PT-DiT block: GIIM then TCM, as five ABI calls.

Order and residuals follow the Qihoo-T2X reading note, code-correspondence
excerpt 2 (PT-Block forward) with Eq. GIIM and Eq. TCM of section 3:
    P  = Averaging(x)                      ptdit_proxy_pool
    P' = P + SA(P)                         ptdit_proxy_sa
    x1 = x + CS(x, P')                     ptdit_proxy_xattn
    x2 = x1 + WSA(x1)                      ptdit_window_sa
    x3 = x2 + SWSA(x2)                     ptdit_shift_window_sa

With caption embeddings (text, [B, L, D]) and MLP weights the rest of the
PT-Block follows (section 3: PT-Block = GIIM + TCM + text cross-attn + MLP):
    x4 = x3 + MHA(x3, text)                ptdit_proxy_xattn (keys/values: text)
    x5 = x4 + MLP(x4)                      ptdit_mlp

Proxy extraction is the window average by default (proxy_mode="mean");
"first" takes each window's top-left token and "random" the token at a
caller-drawn window-local offset (proxy_offsets, int32 [B, M]), the two
alternatives of the pages' proxy-extraction ablation (ptdit_proxy_select).

With bf16 precision the block input is bf16, the residual stream
(P, P', x1, x2, x3) is kept in fp32 and every projection reads its operand
rounded to bf16; x1 and x2 also get a bf16 copy from the epilogue that
writes them, which the next call's Q/K/V projection reads (same values,
half the bytes). With fp32 precision everything is fp32. Buffers and the
workspace are allocated once, in the constructor; forward() only launches.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from . import _lib
from ._lib import AttnWeights, MlpWeights


class PTBlockAttention:
    def __init__(self, B: int, grid: Sequence[int], D: int, heads: int, p: Sequence[int],
                 win: Sequence[int], shift: Sequence[int], weights: Sequence[dict],
                 prec: torch.dtype = torch.bfloat16, device="cuda", proxy_mode: str = "mean",
                 proxy_offsets: Optional[torch.Tensor] = None, text: Optional[torch.Tensor] = None,
                 text_weights: Optional[dict] = None, mlp_weights: Optional[dict] = None):
        self.B = B
        self.F, self.H, self.W = grid
        self.D, self.heads = D, heads
        self.p, self.win, self.shift = tuple(p), tuple(win), tuple(shift)
        self.prec = prec
        self.device = torch.device(device)
        if proxy_mode not in ("mean", "first", "random"):
            raise ValueError(f"proxy_mode {proxy_mode!r}")
        if (proxy_mode == "random") != (proxy_offsets is not None):
            raise ValueError("proxy_offsets go with proxy_mode='random' (and only with it)")
        self.proxy_mode = proxy_mode
        self.proxy_offsets = (proxy_offsets.to(device=self.device, dtype=torch.int32).contiguous()
                              if proxy_offsets is not None else None)
        self.N = self.F * self.H * self.W
        self.M = (self.F // p[0]) * (self.H // p[1]) * (self.W // p[2])
        self.g = (B, self.F, self.H, self.W, D, heads)
        self.weights = [AttnWeights.from_dict(w, prec, self.device) for w in weights]
        # the window attentions' w_qkv packed once for their fused kernel, so
        # a forward launches no packing; after changing the weights in place
        # (an optimizer step), call repack_weights()
        self.repack_weights()
        stream_dt = torch.float32
        self.P = torch.empty(B, self.M, D, dtype=stream_dt, device=self.device)
        self.P2 = torch.empty_like(self.P)
        self.x1 = torch.empty(B, self.N, D, dtype=stream_dt, device=self.device)
        self.x2 = torch.empty_like(self.x1)
        self.x3 = torch.empty_like(self.x1)
        lowp = prec == torch.bfloat16
        self.x1_lowp = torch.empty(B, self.N, D, dtype=torch.bfloat16, device=self.device) if lowp else None
        self.x2_lowp = torch.empty_like(self.x1_lowp) if lowp else None
        if (text is None) != (text_weights is None) or (text is None) != (mlp_weights is None):
            raise ValueError("text, text_weights and mlp_weights go together")
        self.full = text is not None
        need = [
            _lib.workspace_bytes(_lib.OP_PROXY_SA, (B, 1, 1, self.M, D, heads), self.M, (1, 1, 1), prec),
            _lib.workspace_bytes(_lib.OP_PROXY_XATTN, self.g, self.M, (1, 1, 1), prec),
            _lib.workspace_bytes(_lib.OP_WINDOW_SA, self.g, 0, self.win, prec),
        ]
        if self.full:
            self.text = torch.as_tensor(text).to(device=self.device, dtype=prec).contiguous()
            self.L = self.text.shape[1]
            self.w_text = AttnWeights.from_dict(text_weights, prec, self.device)
            self.w_mlp = MlpWeights.from_dict(mlp_weights, prec, self.device)
            self.hidden = self.w_mlp.hidden
            self.x4 = torch.empty_like(self.x1)
            self.x5 = torch.empty_like(self.x1)
            self.x3_lowp = torch.empty_like(self.x1_lowp) if lowp else None
            self.x4_lowp = torch.empty_like(self.x1_lowp) if lowp else None
            need += [_lib.workspace_bytes(_lib.OP_PROXY_XATTN, self.g, self.L, (1, 1, 1), prec),
                     _lib.workspace_bytes(_lib.OP_MLP, (B * self.N, 1, 1, 1, D, 1), self.hidden, (1, 1, 1), prec)]
        self._ws_need = list(need[:3])
        need = max(need)
        self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        self._kws = None     # per-call workspaces of keep mode (allocated on first use)
        self.kept = None     # views of what the last keep-mode forward left for the backward

    def repack_weights(self) -> None:
        """Rewrite the packed copies of the two window attentions' w_qkv
        (ptdit_pack_window_weights) from the current weights. The window calls
        read the packed copy, not w_qkv, so it must follow every in-place
        change of the weights."""
        for w in self.weights[2:4]:
            w.w_qkv_packed = _lib.pack_window_weights(w, self.heads)

    def forward(self, x: torch.Tensor, keep: bool = False) -> torch.Tensor:
        """One forward. keep=True (training): every attention call gets its own
        workspace and the window attentions run as ptdit_window_sa_keep, so the
        Q/K/V and attention outputs of all four attentions stay for the
        backward (self.kept) instead of being recomputed."""
        g, w = self.g, self.weights
        if keep:
            if self._kws is None:
                n_sa, n_x, n_w = self._ws_need
                self._kws = [torch.empty(n, dtype=torch.uint8, device=self.device) for n in (n_sa, n_x, n_w, n_w)]
            ws_sa, ws_x, ws_w, ws_s = self._kws
        else:
            ws_sa = ws_x = ws_w = ws_s = self.ws
        if self.proxy_mode == "mean":
            _lib.proxy_pool(x, g, self.p, out=self.P)
        else:
            _lib.proxy_select(x, g, self.p, self.proxy_offsets, out=self.P)
        _lib.proxy_sa(self.P, self.heads, w[0], residual=True, ws=ws_sa, out=self.P2)
        _lib.proxy_xattn(x, g, self.P2, w[1], residual=True, ws=ws_x, out=self.x1, out_lowp=self.x1_lowp)
        if keep:
            _lib.window_sa_keep(self.x1, g, self.win, (0, 0, 0), w[2], ws_w, residual=True, out=self.x2,
                                x_lowp=self.x1_lowp, out_lowp=self.x2_lowp)
            _lib.window_sa_keep(self.x2, g, self.win, self.shift, w[3], ws_s, residual=True, out=self.x3,
                                x_lowp=self.x2_lowp, out_lowp=self.x3_lowp if self.full else None)
            self.kept = self._kept_views()
        else:
            self.kept = None
            _lib.window_sa(self.x1, g, self.win, w[2], residual=True, ws=self.ws, out=self.x2,
                           x_lowp=self.x1_lowp, out_lowp=self.x2_lowp)
            _lib.shift_window_sa(self.x2, g, self.win, self.shift, w[3], residual=True, ws=self.ws, out=self.x3,
                                 x_lowp=self.x2_lowp, out_lowp=self.x3_lowp if self.full else None)
        if not self.full:
            return self.x3
        _lib.proxy_xattn(self.x3, g, self.text, self.w_text, residual=True, ws=self.ws, out=self.x4,
                         out_lowp=self.x4_lowp, x_lowp=self.x3_lowp)
        _lib.mlp(self.x4, self.w_mlp, residual=True, ws=self.ws, out=self.x5, x_lowp=self.x4_lowp)
        return self.x5

    def _kept_views(self) -> Dict[str, torch.Tensor]:
        """Views of the keep-mode workspaces in the layouts the calls document:
        proxy SA [Q/K/V head-major | O], cross-attention [Q | K/V head-major |
        O], window attentions [Q/K/V head-major | O], each part 256-byte
        aligned."""
        B, N, M, D, heads, prec = self.B, self.N, self.M, self.D, self.heads, self.prec
        dh = D // heads
        es = torch.tensor([], dtype=prec).element_size()
        al = lambda n: (n + 255) // 256 * 256
        part = lambda ws, off, n, shape: ws[off:off + n * es].view(prec).view(*shape)
        ws_sa, ws_x, ws_w, ws_s = self._kws
        out = {"sa_qkv": part(ws_sa, 0, B * 3 * M * D, (B, 3, heads, M, dh)),
               "sa_o": part(ws_sa, al(B * 3 * M * D * es), B * M * D, (B, M, D)),
               "x_q": part(ws_x, 0, B * N * D, (B, 1, heads, N, dh))}
        kv_off = al(B * N * D * es)
        out["x_kv"] = part(ws_x, kv_off, B * 2 * M * D, (B, 2, heads, M, dh))
        out["x_o"] = part(ws_x, kv_off + al(B * 2 * M * D * es), B * N * D, (B, N, D))
        out["wsa_qkv"], out["wsa_o"] = _lib.window_ws_views(ws_w, self.g, prec)
        out["swsa_qkv"], out["swsa_o"] = _lib.window_ws_views(ws_s, self.g, prec)
        return out

    def intermediates(self) -> Dict[str, torch.Tensor]:
        out = {"P": self.P, "P2": self.P2, "x1": self.x1, "x2": self.x2, "x3": self.x3}
        if self.full:
            out.update(x4=self.x4, x5=self.x5)
        return out

    def flops(self) -> Dict[str, int]:
        """Algorithmic FLOPs of one forward (2 per multiply-accumulate): the
        ten projections over real rows plus the four attention cores counted
        dense over their (padded) windows, queries restricted to real tokens."""
        B, N, M, D = self.B, self.N, self.M, self.D
        L = self.win[0] * self.win[1] * self.win[2]
        proj = B * D * D * ((3 * M + M) + (N + 2 * M + N) + 2 * (3 * N + N))
        core = B * D * (2 * M * M + 2 * N * M + 2 * (2 * N * L))
        out = {"projection": 2 * proj, "core": 2 * core, "total": 2 * (proj + core)}
        if getattr(self, "full", False):
            T, Hm = self.L, self.hidden
            text = B * D * (D * (N + 2 * T + N) + 2 * N * T)   # Q, K/V, O maps; Q K^T and P V
            mlp = B * N * D * Hm * 2
            out.update(text=2 * text, mlp=2 * mlp, total=out["total"] + 2 * (text + mlp))
        return out
