"""ctypes binding of libptdit.so (include/ptdit.h).

Argument marshalling only: every operation runs in the HIP kernels behind
the C ABI. torch supplies device memory (data_ptr) and the current HIP
stream. There is no CPU fallback: if the library is missing, loading fails
loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libptdit.so")

PTDIT_BF16, PTDIT_F32 = 0, 1
OP_PROXY_SA, OP_PROXY_XATTN, OP_WINDOW_SA, OP_SHIFT_WINDOW_SA, OP_MLP = 0, 1, 2, 3, 4
(K_POOL, K_GEMM_QKV, K_GEMM_OUT, K_ATTN_FLASH, K_ATTN_WINDOW, K_ROLL, K_GEMM_Q, K_GEMM_PROXY, K_GEMM_MLP,
 K_BWD_WINDOW, K_BWD_DENSE, K_BWD_POOL, K_BWD_LINEAR) = range(13)

STATUS = {0: "PTDIT_OK", -1: "PTDIT_ERR_NULL", -2: "PTDIT_ERR_SHAPE", -3: "PTDIT_ERR_DIVISIBILITY",
          -4: "PTDIT_ERR_DTYPE", -5: "PTDIT_ERR_ALIGN", -6: "PTDIT_ERR_WORKSPACE",
          -7: "PTDIT_ERR_HIP", -8: "PTDIT_ERR_ALIAS"}

EXPORTED = ["ptdit_linear", "ptdit_mlp", "ptdit_proxy_pool", "ptdit_proxy_select", "ptdit_proxy_sa", "ptdit_proxy_xattn",
            "ptdit_window_sa", "ptdit_shift_window_sa", "ptdit_roll3d", "ptdit_workspace_bytes",
            "ptdit_status_str", "ptdit_version", "ptdit_trace_enable", "ptdit_trace_read",
            "ptdit_trace_disable", "ptdit_window_attn_bwd", "ptdit_attn_bwd", "ptdit_attn_bwd_workspace_bytes",
            "ptdit_proxy_pool_bwd", "ptdit_linear_bwd", "ptdit_linear_bwd_workspace_bytes"]


class Grid(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("F", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W", ctypes.c_int32), ("D", ctypes.c_int32), ("heads", ctypes.c_int32)]


class Win3(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class AttnW(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("b_o", ctypes.c_void_p)]


class MlpW(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


class PtditError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libptdit.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with "
                           "`python -m diffusion_transformer_attention_pt_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    G, W3, AW, MW = Grid, Win3, ctypes.POINTER(AttnW), ctypes.POINTER(MlpW)
    sig = {
        "ptdit_linear": [vp, i32, i64, i32, i32, vp, vp, vp, i32, vp, i32, i32, vp],
        "ptdit_proxy_pool": [vp, i32, G, W3, vp, i32, vp],
        "ptdit_proxy_select": [vp, i32, G, W3, vp, vp, i32, vp],
        "ptdit_mlp": [vp, vp, i32, i64, i32, i32, MW, i32, vp, vp, i32, vp, sz, i32, vp],
        "ptdit_proxy_sa": [vp, i32, i32, i32, i32, i32, AW, i32, vp, i32, vp, sz, i32, vp],
        "ptdit_proxy_xattn": [vp, vp, i32, G, vp, i32, i32, AW, i32, vp, vp, i32, vp, sz, i32, vp],
        "ptdit_window_sa": [vp, vp, i32, G, W3, AW, i32, vp, vp, i32, vp, sz, i32, vp],
        "ptdit_shift_window_sa": [vp, vp, i32, G, W3, W3, AW, i32, vp, vp, i32, vp, sz, i32, vp],
        "ptdit_roll3d": [vp, G, W3, i32, vp, i32, vp],
        "ptdit_workspace_bytes": [i32, G, i32, W3, i32],
        "ptdit_status_str": [i32],
        "ptdit_version": [],
        "ptdit_trace_enable": [i32, i32],
        "ptdit_trace_read": [ctypes.POINTER(ctypes.c_float), i32],
        "ptdit_trace_disable": [],
        "ptdit_window_attn_bwd": [vp, vp, vp, i32, G, W3, W3, vp, vp, vp],
        "ptdit_attn_bwd": [vp, i64, vp, vp, i64, vp, i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i64, vp, sz, vp],
        "ptdit_attn_bwd_workspace_bytes": [i32, i32, i32, i32, i32],
        "ptdit_proxy_pool_bwd": [vp, G, W3, vp, i32, vp],
        "ptdit_linear_bwd": [vp, i32, i64, i32, i32, vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "ptdit_linear_bwd_workspace_bytes": [i64, i32, i32],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = i32
    lib.ptdit_workspace_bytes.restype = sz
    lib.ptdit_attn_bwd_workspace_bytes.restype = sz
    lib.ptdit_linear_bwd_workspace_bytes.restype = sz
    lib.ptdit_status_str.restype = ctypes.c_char_p
    lib.ptdit_version.restype = ctypes.c_char_p
    lib.ptdit_trace_disable.restype = None
    _lib = lib
    return lib


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return PTDIT_BF16
    if t == torch.float32:
        return PTDIT_F32
    raise TypeError(f"unsupported dtype {t}")


def _tdt(code: int) -> torch.dtype:
    return torch.bfloat16 if code == PTDIT_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise PtditError(fn, st)


@dataclass
class AttnWeights:
    """Weights of one attention module in the ABI layout: w_qkv [3D, D]
    (W_q rows, then W_k, then W_v), b_qkv [3D], w_o [D, D], b_o [D]."""
    w_qkv: torch.Tensor
    b_qkv: Optional[torch.Tensor]
    w_o: torch.Tensor
    b_o: Optional[torch.Tensor]

    @staticmethod
    def from_dict(w: dict, dtype: torch.dtype, device) -> "AttnWeights":
        t = lambda a: torch.as_tensor(a).to(device=device, dtype=dtype).contiguous()
        wqkv = torch.cat([t(w["wq"]), t(w["wk"]), t(w["wv"])], 0).contiguous()
        b = None
        if w.get("bq") is not None:
            b = torch.cat([t(w["bq"]), t(w["bk"]), t(w["bv"])], 0).contiguous()
        return AttnWeights(wqkv, b, t(w["wo"]), t(w["bo"]) if w.get("bo") is not None else None)

    @property
    def dtype(self) -> torch.dtype:
        return self.w_qkv.dtype

    def c(self) -> AttnW:
        return AttnW(_ptr(self.w_qkv), _ptr(self.b_qkv), _ptr(self.w_o), _ptr(self.b_o))


@dataclass
class MlpWeights:
    """Weights of the MLP in the ABI layout: w1 [H, D], b1 [H], w2 [D, H], b2 [D]."""
    w1: torch.Tensor
    b1: Optional[torch.Tensor]
    w2: torch.Tensor
    b2: Optional[torch.Tensor]

    @staticmethod
    def from_dict(w: dict, dtype: torch.dtype, device) -> "MlpWeights":
        t = lambda a: torch.as_tensor(a).to(device=device, dtype=dtype).contiguous()
        return MlpWeights(t(w["w1"]), t(w["b1"]) if w.get("b1") is not None else None,
                          t(w["w2"]), t(w["b2"]) if w.get("b2") is not None else None)

    @property
    def dtype(self) -> torch.dtype:
        return self.w1.dtype

    @property
    def hidden(self) -> int:
        return self.w1.shape[0]

    def c(self) -> MlpW:
        return MlpW(_ptr(self.w1), _ptr(self.b1), _ptr(self.w2), _ptr(self.b2))


def mlp(x: torch.Tensor, w: MlpWeights, residual: bool = True, out_dtype: Optional[torch.dtype] = None,
        ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
        x_lowp: Optional[torch.Tensor] = None, out_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [..., D] -> Lin(GELU(Lin(x; w1, b1)); w2, b2) (+ x)."""
    lib = load()
    D = x.shape[-1]
    rows = x.numel() // D
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    need = workspace_bytes(OP_MLP, (rows, 1, 1, 1, D, 1), w.hidden, (1, 1, 1), w.dtype)
    ws = _ws(need, ws, x.device)
    cw = w.c()
    st = lib.ptdit_mlp(_ptr(x), _ptr(x_lowp), _dt(x.dtype), rows, D, w.hidden, ctypes.byref(cw), int(residual),
                       _ptr(out), _ptr(out_lowp), _dt(out.dtype), _ptr(ws), ws.numel(), _dt(w.dtype), _stream())
    _check("ptdit_mlp", st)
    return out


def version() -> str:
    return load().ptdit_version().decode()


def workspace_bytes(op: int, grid: Sequence[int], M: int, win: Sequence[int], prec: torch.dtype) -> int:
    return int(load().ptdit_workspace_bytes(op, Grid(*grid), M, Win3(*win), _dt(prec)))


def _ws(nbytes: int, ws: Optional[torch.Tensor], device) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def linear(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor] = None,
           residual: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    rows = x.numel() // x.shape[-1]
    d_in, d_out = x.shape[-1], w.shape[0]
    if out is None:
        out = torch.empty(*x.shape[:-1], d_out, dtype=out_dtype or x.dtype, device=x.device)
    r_dt = _dt(residual.dtype) if residual is not None else _dt(out.dtype)
    st = lib.ptdit_linear(_ptr(x), _dt(x.dtype), rows, d_in, d_out, _ptr(w), _ptr(b), _ptr(residual),
                          r_dt, _ptr(out), _dt(out.dtype), _dt(w.dtype), _stream())
    _check("ptdit_linear", st)
    return out


def proxy_select(x: torch.Tensor, grid: Sequence[int], p: Sequence[int],
                 offsets: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grid = (B, F, H, W, D, heads); x [B, N, D] -> proxies [B, M, D], one
    token per window (offsets: int32 [B, M] window-local offsets, or None for
    the top-left token)."""
    lib = load()
    B, F, H, W, D, _ = grid
    M = (F // p[0]) * (H // p[1]) * (W // p[2]) if all(p) else 0
    if offsets is not None:
        if offsets.dtype != torch.int32 or offsets.numel() != B * M:
            raise ValueError("offsets must be int32 [B, M]")
    if out is None:
        out = torch.empty(B, M, D, dtype=out_dtype or x.dtype, device=x.device)
    st = lib.ptdit_proxy_select(_ptr(x), _dt(x.dtype), Grid(*grid), Win3(*p), _ptr(offsets), _ptr(out),
                                _dt(out.dtype), _stream())
    _check("ptdit_proxy_select", st)
    return out


def proxy_pool(x: torch.Tensor, grid: Sequence[int], p: Sequence[int],
               out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grid = (B, F, H, W, D, heads); x [B, N, D] -> proxies [B, M, D]."""
    lib = load()
    B, F, H, W, D, _ = grid
    M = (F // p[0]) * (H // p[1]) * (W // p[2]) if all(p) else 0
    if out is None:
        out = torch.empty(B, M, D, dtype=out_dtype or x.dtype, device=x.device)
    st = lib.ptdit_proxy_pool(_ptr(x), _dt(x.dtype), Grid(*grid), Win3(*p), _ptr(out), _dt(out.dtype),
                              _stream())
    _check("ptdit_proxy_pool", st)
    return out


def proxy_sa(P: torch.Tensor, heads: int, w: AttnWeights, residual: bool = True,
             out_dtype: Optional[torch.dtype] = None, ws: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    B, M, D = P.shape
    if out is None:
        out = torch.empty(B, M, D, dtype=out_dtype or P.dtype, device=P.device)
    need = workspace_bytes(OP_PROXY_SA, (B, 1, 1, M, D, heads), M, (1, 1, 1), w.dtype)
    ws = _ws(need, ws, P.device)
    cw = w.c()
    st = lib.ptdit_proxy_sa(_ptr(P), _dt(P.dtype), B, M, D, heads, ctypes.byref(cw), int(residual),
                            _ptr(out), _dt(out.dtype), _ptr(ws), ws.numel(), _dt(w.dtype), _stream())
    _check("ptdit_proxy_sa", st)
    return out


def proxy_xattn(x: torch.Tensor, grid: Sequence[int], P2: torch.Tensor, w: AttnWeights,
                residual: bool = True, out_dtype: Optional[torch.dtype] = None,
                ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                out_lowp: Optional[torch.Tensor] = None, x_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out_lowp: optional bf16 tensor of out's shape that receives bf16(out);
    x_lowp: optional bf16 copy of an fp32 x, read by the query projection."""
    lib = load()
    M = P2.shape[1]
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    need = workspace_bytes(OP_PROXY_XATTN, grid, M, (1, 1, 1), w.dtype)
    ws = _ws(need, ws, x.device)
    cw = w.c()
    st = lib.ptdit_proxy_xattn(_ptr(x), _ptr(x_lowp), _dt(x.dtype), Grid(*grid), _ptr(P2), _dt(P2.dtype), M,
                               ctypes.byref(cw), int(residual), _ptr(out), _ptr(out_lowp), _dt(out.dtype),
                               _ptr(ws), ws.numel(), _dt(w.dtype), _stream())
    _check("ptdit_proxy_xattn", st)
    return out


def window_sa(x: torch.Tensor, grid: Sequence[int], win: Sequence[int], w: AttnWeights,
              residual: bool = True, out_dtype: Optional[torch.dtype] = None,
              ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              x_lowp: Optional[torch.Tensor] = None, out_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_lowp: optional bf16 copy of an fp32 x (read by the projection);
    out_lowp: optional bf16 tensor that receives bf16(out)."""
    lib = load()
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    need = workspace_bytes(OP_WINDOW_SA, grid, 0, win, w.dtype)
    ws = _ws(need, ws, x.device)
    cw = w.c()
    st = lib.ptdit_window_sa(_ptr(x), _ptr(x_lowp), _dt(x.dtype), Grid(*grid), Win3(*win),
                             ctypes.byref(cw), int(residual), _ptr(out), _ptr(out_lowp), _dt(out.dtype),
                             _ptr(ws), ws.numel(), _dt(w.dtype), _stream())
    _check("ptdit_window_sa", st)
    return out


def shift_window_sa(x: torch.Tensor, grid: Sequence[int], win: Sequence[int], shift: Sequence[int],
                    w: AttnWeights, residual: bool = True, out_dtype: Optional[torch.dtype] = None,
                    ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    x_lowp: Optional[torch.Tensor] = None,
                    out_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_lowp / out_lowp as for window_sa."""
    lib = load()
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    need = workspace_bytes(OP_SHIFT_WINDOW_SA, grid, 0, win, w.dtype)
    ws = _ws(need, ws, x.device)
    cw = w.c()
    st = lib.ptdit_shift_window_sa(_ptr(x), _ptr(x_lowp), _dt(x.dtype), Grid(*grid), Win3(*win),
                                   Win3(*shift), ctypes.byref(cw), int(residual), _ptr(out),
                                   _ptr(out_lowp), _dt(out.dtype), _ptr(ws), ws.numel(), _dt(w.dtype),
                                   _stream())
    _check("ptdit_shift_window_sa", st)
    return out


def roll3d(x: torch.Tensor, grid: Sequence[int], shift: Sequence[int], inverse: bool = False,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    if out is None:
        out = torch.empty_like(x)
    st = lib.ptdit_roll3d(_ptr(x), Grid(*grid), Win3(*shift), int(inverse), _ptr(out), _dt(x.dtype),
                          _stream())
    _check("ptdit_roll3d", st)
    return out


def window_attn_bwd(qkv: torch.Tensor, d_o: torch.Tensor, grid: Sequence[int], win: Sequence[int],
                    shift: Sequence[int] = (0, 0, 0), b_qkv: Optional[torch.Tensor] = None,
                    d_qkv: Optional[torch.Tensor] = None, d_b_kv: Optional[torch.Tensor] = None):
    """Backward of the window / shifted-window attention core. qkv [B, 3, heads,
    N, dh] (the forward's Q/K/V), d_o [B, N, D]. Returns (d_qkv fp32 [B, 3, heads,
    N, dh], d_b_kv fp32 [2, D]: pad-slot gradients, added to d_b_kv when given)."""
    lib = load()
    B, F, H, W, D, heads = grid
    if d_o.dtype != qkv.dtype or (b_qkv is not None and b_qkv.dtype != qkv.dtype):
        raise ValueError("qkv, d_o and b_qkv must share one dtype")
    if d_qkv is None:
        d_qkv = torch.empty(qkv.shape, dtype=torch.float32, device=qkv.device)
    if d_b_kv is None:
        d_b_kv = torch.zeros(2, D, dtype=torch.float32, device=qkv.device)
    st = lib.ptdit_window_attn_bwd(_ptr(qkv), _ptr(b_qkv), _ptr(d_o), _dt(qkv.dtype), Grid(*grid), Win3(*win),
                                   Win3(*shift), _ptr(d_qkv), _ptr(d_b_kv), _stream())
    _check("ptdit_window_attn_bwd", st)
    return d_qkv, d_b_kv


def _bhld(t: torch.Tensor, name: str) -> int:
    """Batch stride (elements) of a [B, heads, L, dh] view whose batch items are contiguous."""
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must live on the GPU")
    B, h, L, dh = t.shape
    if t.stride(3) != 1 or t.stride(2) != dh or t.stride(1) != L * dh:
        raise ValueError(f"{name}: each batch item must be a contiguous [heads, L, dh] block")
    return t.stride(0)


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, d_o: torch.Tensor,
             ws: Optional[torch.Tensor] = None):
    """Backward of the unmasked attention core (proxy SA, cross-attention).
    q [B, heads, Nq, dh], k / v [B, heads, Nk, dh] (views into fused buffers
    allowed), d_o [B, Nq, heads*dh]. Returns fp32 (dq, dk, dv), contiguous."""
    lib = load()
    B, heads, Nq, dh = q.shape
    Nk = k.shape[2]
    if k.stride(0) != v.stride(0):
        raise ValueError("k and v must share their batch stride")
    dq = torch.empty(B, heads, Nq, dh, dtype=torch.float32, device=q.device)
    dk = torch.empty(B, heads, Nk, dh, dtype=torch.float32, device=q.device)
    dv = torch.empty(B, heads, Nk, dh, dtype=torch.float32, device=q.device)
    need = int(lib.ptdit_attn_bwd_workspace_bytes(B, heads, Nq, Nk, dh))
    ws = _ws(need, ws, q.device)
    if len({q.dtype, k.dtype, v.dtype, d_o.dtype}) != 1:
        raise ValueError("q, k, v and d_o must share one dtype")
    q_bs, kv_bs = _bhld(q, "q"), _bhld(k, "k")
    _bhld(v, "v")
    st = lib.ptdit_attn_bwd(q.data_ptr(), q_bs, k.data_ptr(), v.data_ptr(), kv_bs, _ptr(d_o), _dt(q.dtype),
                            B, heads, Nq, Nk, dh, _ptr(dq), heads * Nq * dh, _ptr(dk), _ptr(dv), heads * Nk * dh,
                            _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check("ptdit_attn_bwd", st)
    return dq, dk, dv


def proxy_pool_bwd(d_proxies: torch.Tensor, grid: Sequence[int], p: Sequence[int],
                   d_x: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """Backward of the window average: d_x[token] (+)= d_proxies[its proxy] / P (fp32)."""
    lib = load()
    B, F, H, W, D, _ = grid
    if d_x is None:
        d_x = torch.empty(B, F * H * W, D, dtype=torch.float32, device=d_proxies.device)
    st = lib.ptdit_proxy_pool_bwd(_ptr(d_proxies), Grid(*grid), Win3(*p), _ptr(d_x), int(accumulate), _stream())
    _check("ptdit_proxy_pool_bwd", st)
    return d_x


def linear_bwd(x: torch.Tensor, w: torch.Tensor, d_y: torch.Tensor, want_dx: bool = True, want_dw: bool = True,
               want_db: bool = True, ws: Optional[torch.Tensor] = None):
    """Gradients of Y = X W^T + b: x [..., d_in], w [d_out, d_in] bf16, d_y [..., d_out].
    Returns fp32 (d_x or None, d_w or None, d_b or None)."""
    lib = load()
    d_in, d_out = x.shape[-1], w.shape[0]
    rows = x.numel() // d_in
    dev = x.device
    dx = torch.empty(*x.shape[:-1], d_in, dtype=torch.float32, device=dev) if want_dx else None
    dw = torch.empty(d_out, d_in, dtype=torch.float32, device=dev) if want_dw else None
    db = torch.empty(d_out, dtype=torch.float32, device=dev) if want_db else None
    need = int(lib.ptdit_linear_bwd_workspace_bytes(rows, d_in, d_out))
    ws = _ws(need, ws, dev)
    st = lib.ptdit_linear_bwd(_ptr(x), _dt(x.dtype), rows, d_in, d_out, _ptr(w), _ptr(d_y), _dt(d_y.dtype),
                              _ptr(dx), _ptr(dw), _ptr(db), _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check("ptdit_linear_bwd", st)
    return dx, dw, db


def trace_enable(kernel_class: int, capacity: int) -> None:
    _check("ptdit_trace_enable", load().ptdit_trace_enable(kernel_class, capacity))


def trace_read(max_n: int) -> list:
    buf = (ctypes.c_float * max_n)()
    n = load().ptdit_trace_read(buf, max_n)
    return [buf[i] for i in range(n)]


def trace_disable() -> None:
    load().ptdit_trace_disable()
