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
 K_BWD_WINDOW, K_BWD_DENSE, K_BWD_POOL, K_BWD_LINEAR, K_WINDOW_FUSED) = range(14)

STATUS = {0: "PTDIT_OK", -1: "PTDIT_ERR_NULL", -2: "PTDIT_ERR_SHAPE", -3: "PTDIT_ERR_DIVISIBILITY",
          -4: "PTDIT_ERR_DTYPE", -5: "PTDIT_ERR_ALIGN", -6: "PTDIT_ERR_WORKSPACE",
          -7: "PTDIT_ERR_HIP", -8: "PTDIT_ERR_ALIAS", -9: "PTDIT_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # PTDIT_NOALLOC_SCRATCH_BYTES

EXPORTED = ["ptdit_linear", "ptdit_mlp", "ptdit_proxy_pool", "ptdit_proxy_select", "ptdit_proxy_sa", "ptdit_proxy_sa_noalloc", "ptdit_proxy_xattn",
            "ptdit_window_sa", "ptdit_shift_window_sa", "ptdit_roll3d", "ptdit_workspace_bytes",
            "ptdit_status_str", "ptdit_version", "ptdit_trace_enable", "ptdit_trace_read",
            "ptdit_trace_disable", "ptdit_window_attn_bwd", "ptdit_attn_bwd", "ptdit_attn_bwd_workspace_bytes",
            "ptdit_proxy_pool_bwd", "ptdit_linear_bwd", "ptdit_linear_bwd_workspace_bytes",
            "ptdit_linear_heads", "ptdit_window_attn", "ptdit_attn", "ptdit_attn_workspace_bytes",
            "ptdit_heads_to_tokens", "ptdit_f32_to_bf16", "ptdit_add_f32", "ptdit_calibrate_mfma",
            "ptdit_calibrate_read", "ptdit_calibrate_copy", "ptdit_linear_bwd_ex",
            "ptdit_window_attn_bwd_tokens", "ptdit_window_sa_keep", "ptdit_attn_bwd_tokens",
            "ptdit_window_packed_bytes", "ptdit_pack_window_weights", "ptdit_linear_bwd_dw_group",
            "ptdit_linear_bwd_dw_group_workspace_bytes"]


class Grid(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("F", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W", ctypes.c_int32), ("D", ctypes.c_int32), ("heads", ctypes.c_int32)]


class Win3(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class AttnW(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("b_o", ctypes.c_void_p), ("w_qkv_packed", ctypes.c_void_p)]


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
        "ptdit_proxy_sa_noalloc": [vp, i32, i32, i32, i32, i32, AW, i32, vp, i32, i32, vp],
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
        "ptdit_window_attn_bwd_tokens": [vp, vp, vp, i32, G, W3, W3, vp, i32, vp, vp],
        "ptdit_window_sa_keep": [vp, vp, i32, G, W3, W3, AW, i32, vp, vp, i32, vp, sz, i32, vp],
        "ptdit_attn_bwd": [vp, i64, vp, vp, i64, vp, i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i64, vp, sz, vp],
        "ptdit_attn_bwd_tokens": [vp, i64, vp, vp, i64, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, i64, vp,
                                  sz, vp],
        "ptdit_attn_bwd_workspace_bytes": [i32, i32, i32, i32, i32],
        "ptdit_proxy_pool_bwd": [vp, G, W3, vp, i32, vp],
        "ptdit_linear_bwd": [vp, i32, i64, i32, i32, vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "ptdit_linear_bwd_ex": [vp, i32, i64, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp],
        "ptdit_linear_bwd_workspace_bytes": [i64, i32, i32],
        "ptdit_linear_heads": [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp],
        "ptdit_window_attn": [vp, vp, i32, G, W3, W3, vp, vp],
        "ptdit_attn": [vp, i64, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp],
        "ptdit_attn_workspace_bytes": [i32, i32, i32, i32],
        "ptdit_heads_to_tokens": [vp, i32, i32, i32, i32, i32, vp, vp],
        "ptdit_f32_to_bf16": [vp, i64, vp, vp],
        "ptdit_add_f32": [vp, vp, i64, vp, vp],
        "ptdit_calibrate_mfma": [i32, i32, vp, ctypes.POINTER(ctypes.c_int64), vp],
        "ptdit_calibrate_read": [vp, i64, i32, vp, vp],
        "ptdit_calibrate_copy": [vp, vp, i64, vp],
        "ptdit_window_packed_bytes": [i32, i32],
        "ptdit_pack_window_weights": [vp, i32, i32, vp, vp],
        "ptdit_linear_bwd_dw_group": [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i32, i32,
                                      ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp],
        "ptdit_linear_bwd_dw_group_workspace_bytes": [i32, i64, i32, i32],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = i32
    lib.ptdit_workspace_bytes.restype = sz
    lib.ptdit_attn_bwd_workspace_bytes.restype = sz
    lib.ptdit_linear_bwd_workspace_bytes.restype = sz
    lib.ptdit_attn_workspace_bytes.restype = sz
    lib.ptdit_window_packed_bytes.restype = sz
    lib.ptdit_linear_bwd_dw_group_workspace_bytes.restype = sz
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


def _numel(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """Raise before any launch when a tensor's element count differs from
    what the grid says it holds (the kernels index by the grid)."""
    if t is not None and t.numel() != n:
        raise ValueError(f"{name}: {tuple(t.shape)} holds {t.numel()} elements, the grid needs {n}")


def _proxy_count(grid: Sequence[int], p: Sequence[int]) -> Optional[int]:
    """B*M*D elements of the proxies, or None when p does not divide the grid
    (the library then reports PTDIT_ERR_DIVISIBILITY itself)."""
    B, F, H, W, D, _ = grid
    if not all(p) or F % p[0] or H % p[1] or W % p[2]:
        return None
    return B * (F // p[0]) * (H // p[1]) * (W // p[2]) * D


def _weights(w: "AttnWeights", D: int) -> None:
    if tuple(w.w_qkv.shape) != (3 * D, D) or tuple(w.w_o.shape) != (D, D):
        raise ValueError(f"attention weights must be w_qkv [{3 * D}, {D}] and w_o [{D}, {D}]")
    _numel(w.b_qkv, 3 * D, "b_qkv")
    _numel(w.b_o, D, "b_o")


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
    # optional: w_qkv packed for the window calls' fused kernel
    # (pack_window_weights); must be repacked whenever w_qkv changes
    w_qkv_packed: Optional[torch.Tensor] = None

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
        return AttnW(_ptr(self.w_qkv), _ptr(self.b_qkv), _ptr(self.w_o), _ptr(self.b_o), _ptr(self.w_qkv_packed))


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
    for t, name in ((out, "out"), (x_lowp, "x_lowp"), (out_lowp, "out_lowp")):
        _numel(t, rows * D, name)
    if tuple(w.w1.shape) != (w.hidden, D) or tuple(w.w2.shape) != (D, w.hidden):
        raise ValueError(f"MLP weights must be w1 [H, {D}] and w2 [{D}, H]")
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
    if tuple(w.shape) != (d_out, d_in):
        raise ValueError(f"w must be [d_out, {d_in}]")
    _numel(b, d_out, "b")
    _numel(residual, rows * d_out, "residual")
    _numel(out, rows * d_out, "out")
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
    _numel(x, B * F * H * W * D, "x")
    if _proxy_count(grid, p) is not None:
        _numel(out, _proxy_count(grid, p), "out")
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
    _numel(x, B * F * H * W * D, "x")
    if _proxy_count(grid, p) is not None:
        _numel(out, _proxy_count(grid, p), "out")
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
    _weights(w, D)
    _numel(out, B * M * D, "out")
    if out is None:
        out = torch.empty(B, M, D, dtype=out_dtype or P.dtype, device=P.device)
    need = workspace_bytes(OP_PROXY_SA, (B, 1, 1, M, D, heads), M, (1, 1, 1), w.dtype)
    ws = _ws(need, ws, P.device)
    cw = w.c()
    st = lib.ptdit_proxy_sa(_ptr(P), _dt(P.dtype), B, M, D, heads, ctypes.byref(cw), int(residual),
                            _ptr(out), _dt(out.dtype), _ptr(ws), ws.numel(), _dt(w.dtype), _stream())
    _check("ptdit_proxy_sa", st)
    return out


def proxy_sa_noalloc(P: torch.Tensor, heads: int, w: AttnWeights, out: torch.Tensor,
                     residual: bool = True) -> torch.Tensor:
    """proxy_sa on the library's static scratch (ptdit_proxy_sa_noalloc): no
    workspace, and nothing allocated here either (the caller passes out)."""
    lib = load()
    B, M, D = P.shape
    _weights(w, D)
    _numel(out, B * M * D, "out")
    cw = w.c()
    st = lib.ptdit_proxy_sa_noalloc(_ptr(P), _dt(P.dtype), B, M, D, heads, ctypes.byref(cw), int(residual),
                                    _ptr(out), _dt(out.dtype), _dt(w.dtype), _stream())
    _check("ptdit_proxy_sa_noalloc", st)
    return out


def proxy_xattn(x: torch.Tensor, grid: Sequence[int], P2: torch.Tensor, w: AttnWeights,
                residual: bool = True, out_dtype: Optional[torch.dtype] = None,
                ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                out_lowp: Optional[torch.Tensor] = None, x_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out_lowp: optional bf16 tensor of out's shape that receives bf16(out);
    x_lowp: optional bf16 copy of an fp32 x, read by the query projection."""
    lib = load()
    B, F, H, W, D, _ = grid
    if P2.dim() != 3 or P2.shape[0] != B or P2.shape[2] != D:
        raise ValueError(f"keys/values must be [{B}, M, {D}]")
    M = P2.shape[1]
    _weights(w, D)
    for t, name in ((x, "x"), (out, "out"), (out_lowp, "out_lowp"), (x_lowp, "x_lowp")):
        _numel(t, B * F * H * W * D, name)
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


def pack_window_weights(w: AttnWeights, heads: int) -> Optional[torch.Tensor]:
    """w_qkv packed in the window calls' fused-kernel load order
    (ptdit_pack_window_weights), or None where that kernel does not apply
    (fp32 weights, head width other than 72, ...). Attach the result as
    w.w_qkv_packed so the window calls skip their per-call packing."""
    lib = load()
    D = w.w_qkv.shape[1]
    nb = int(lib.ptdit_window_packed_bytes(D, heads)) if w.dtype == torch.bfloat16 else 0
    if nb == 0:
        return None
    out = torch.empty(nb // 2, dtype=torch.bfloat16, device=w.w_qkv.device)
    st = lib.ptdit_pack_window_weights(_ptr(w.w_qkv), D, heads, _ptr(out), _stream())
    _check("ptdit_pack_window_weights", st)
    return out


def _window_shapes(grid, w, x, out, x_lowp, out_lowp) -> None:
    B, F, H, W, D, _ = grid
    _weights(w, D)
    for t, name in ((x, "x"), (out, "out"), (x_lowp, "x_lowp"), (out_lowp, "out_lowp")):
        _numel(t, B * F * H * W * D, name)


def window_sa(x: torch.Tensor, grid: Sequence[int], win: Sequence[int], w: AttnWeights,
              residual: bool = True, out_dtype: Optional[torch.dtype] = None,
              ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              x_lowp: Optional[torch.Tensor] = None, out_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_lowp: optional bf16 copy of an fp32 x (read by the projection);
    out_lowp: optional bf16 tensor that receives bf16(out)."""
    lib = load()
    _window_shapes(grid, w, x, out, x_lowp, out_lowp)
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
    _window_shapes(grid, w, x, out, x_lowp, out_lowp)
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


def window_sa_keep(x: torch.Tensor, grid: Sequence[int], win: Sequence[int], shift: Sequence[int],
                   w: AttnWeights, ws: torch.Tensor, residual: bool = True, out_dtype: Optional[torch.dtype] = None,
                   out: Optional[torch.Tensor] = None, x_lowp: Optional[torch.Tensor] = None,
                   out_lowp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """window_sa (shift (0, 0, 0)) or shift_window_sa that leaves the head-major
    Q/K/V and the attention output in ws (ptdit_window_sa_keep; window_ws_views
    reads them)."""
    lib = load()
    _window_shapes(grid, w, x, out, x_lowp, out_lowp)
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    need = workspace_bytes(OP_WINDOW_SA, grid, 0, win, w.dtype)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"window_sa_keep: the workspace needs {need} bytes")
    cw = w.c()
    st = lib.ptdit_window_sa_keep(_ptr(x), _ptr(x_lowp), _dt(x.dtype), Grid(*grid), Win3(*win), Win3(*shift),
                                  ctypes.byref(cw), int(residual), _ptr(out), _ptr(out_lowp), _dt(out.dtype),
                                  _ptr(ws), ws.numel() * ws.element_size(), _dt(w.dtype), _stream())
    _check("ptdit_window_sa_keep", st)
    return out


def _align(n: int) -> int:
    return (n + 255) // 256 * 256


def window_ws_views(ws: torch.Tensor, grid: Sequence[int], prec: torch.dtype):
    """(qkv [B, 3, heads, N, dh], o [B, N, D]) views of a window call's
    workspace (the layout ptdit_window_sa_keep documents)."""
    B, F, H, W, D, heads = grid
    N = F * H * W
    es = torch.tensor([], dtype=prec).element_size()
    flat = ws.view(torch.uint8).view(-1)
    qkv = flat[:B * 3 * N * D * es].view(prec).view(B, 3, heads, N, D // heads)
    off = _align(B * 3 * N * D * es)
    o = flat[off:off + B * N * D * es].view(prec).view(B, N, D)
    return qkv, o


def roll3d(x: torch.Tensor, grid: Sequence[int], shift: Sequence[int], inverse: bool = False,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    B, F, H, W, D, _ = grid
    _numel(x, B * F * H * W * D, "x")
    _numel(out, B * F * H * W * D, "out")
    if out is None:
        out = torch.empty_like(x)
    st = lib.ptdit_roll3d(_ptr(x), Grid(*grid), Win3(*shift), int(inverse), _ptr(out), _dt(x.dtype),
                          _stream())
    _check("ptdit_roll3d", st)
    return out


def window_attn_bwd(qkv: torch.Tensor, d_o: torch.Tensor, grid: Sequence[int], win: Sequence[int],
                    shift: Sequence[int] = (0, 0, 0), b_qkv: Optional[torch.Tensor] = None,
                    d_qkv: Optional[torch.Tensor] = None, d_b_kv: Optional[torch.Tensor] = None,
                    tokens: bool = False, pad_grad: bool = True):
    """Backward of the window / shifted-window attention core. qkv [B, 3, heads,
    N, dh] (the forward's Q/K/V), d_o [B, N, D]. Returns (d_qkv fp32 [B, 3, heads,
    N, dh], or [B, N, 3D] with tokens=True (ptdit_window_attn_bwd_tokens; then a
    given d_qkv may also be bf16, for bf16 inputs), d_b_kv fp32 [2, D]: pad-slot
    gradients, added to d_b_kv when given). With pad_grad=False and no d_b_kv,
    no pad-slot buffer is made (None is returned in its place): for grids the
    window divides, where the library then reads and writes none (it refuses
    the call otherwise)."""
    lib = load()
    B, F, H, W, D, heads = grid
    if d_o.dtype != qkv.dtype or (b_qkv is not None and b_qkv.dtype != qkv.dtype):
        raise ValueError("qkv, d_o and b_qkv must share one dtype")
    N = F * H * W
    _numel(qkv, B * 3 * N * D, "qkv")
    _numel(d_o, B * N * D, "d_o")
    _numel(b_qkv, 3 * D, "b_qkv")
    _numel(d_qkv, B * 3 * N * D, "d_qkv")
    _numel(d_b_kv, 2 * D, "d_b_kv")
    if d_qkv is None:
        shape = (B, N, 3 * D) if tokens else tuple(qkv.shape)
        d_qkv = torch.empty(shape, dtype=torch.float32, device=qkv.device)
    if d_qkv.dtype != torch.float32 and not (tokens and d_qkv.dtype == torch.bfloat16):
        raise ValueError("d_qkv must be float32 (or bfloat16 with tokens=True)")
    if d_b_kv is None and pad_grad:
        d_b_kv = torch.zeros(2, D, dtype=torch.float32, device=qkv.device)
    if tokens:
        st = lib.ptdit_window_attn_bwd_tokens(_ptr(qkv), _ptr(b_qkv), _ptr(d_o), _dt(qkv.dtype), Grid(*grid),
                                              Win3(*win), Win3(*shift), _ptr(d_qkv), _dt(d_qkv.dtype),
                                              _ptr(d_b_kv), _stream())
    else:
        st = lib.ptdit_window_attn_bwd(_ptr(qkv), _ptr(b_qkv), _ptr(d_o), _dt(qkv.dtype), Grid(*grid), Win3(*win),
                                       Win3(*shift), _ptr(d_qkv), _ptr(d_b_kv), _stream())
    _check("ptdit_window_attn_bwd_tokens" if tokens else "ptdit_window_attn_bwd", st)
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
             ws: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None, dq_tokens: bool = False):
    """Backward of the unmasked attention core (proxy SA, cross-attention).
    q [B, heads, Nq, dh], k / v [B, heads, Nk, dh] (views into fused buffers
    allowed), d_o [B, Nq, heads*dh]. Returns fp32 (dq, dk, dv): new contiguous
    tensors, or the given fp32 views (each batch item a contiguous [heads, L,
    dh] block; dk and dv with one batch stride). dq_tokens: dq token-major
    [B, Nq, heads*dh] (ptdit_attn_bwd_tokens), fp32 or, for bf16 inputs, a
    given bf16 tensor."""
    lib = load()
    B, heads, Nq, dh = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, heads, Nk, dh) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k and v must both be [{B}, {heads}, Nk, {dh}]")
    _numel(d_o, B * Nq * heads * dh, "d_o")
    if k.stride(0) != v.stride(0):
        raise ValueError("k and v must share their batch stride")
    for t, n, name in (((None if dq_tokens else dq), Nq, "dq"), (dk, Nk, "dk"), (dv, Nk, "dv")):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, heads, n, dh)):
            raise ValueError(f"{name} must be fp32 [{B}, {heads}, {n}, {dh}]")
    if dq_tokens and dq is not None:
        if dq.dtype not in (torch.float32, torch.bfloat16) or not dq.is_contiguous():
            raise ValueError("dq (token-major) must be a contiguous fp32 or bf16 tensor")
        _numel(dq, B * Nq * heads * dh, "dq")
    if dq is None:
        dq = torch.empty(*((B, Nq, heads * dh) if dq_tokens else (B, heads, Nq, dh)), dtype=torch.float32,
                         device=q.device)
    if dk is None:
        dk = torch.empty(B, heads, Nk, dh, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(B, heads, Nk, dh, dtype=torch.float32, device=q.device)
    dq_bs = None if dq_tokens else _bhld(dq, "dq")
    dk_bs, dv_bs = _bhld(dk, "dk"), _bhld(dv, "dv")
    if dk_bs != dv_bs:
        raise ValueError("dk and dv must share their batch stride")
    need = int(lib.ptdit_attn_bwd_workspace_bytes(B, heads, Nq, Nk, dh))
    ws = _ws(need, ws, q.device)
    if len({q.dtype, k.dtype, v.dtype, d_o.dtype}) != 1:
        raise ValueError("q, k, v and d_o must share one dtype")
    q_bs, kv_bs = _bhld(q, "q"), _bhld(k, "k")
    _bhld(v, "v")
    if dq_tokens:
        st = lib.ptdit_attn_bwd_tokens(q.data_ptr(), q_bs, k.data_ptr(), v.data_ptr(), kv_bs, _ptr(d_o),
                                       _dt(q.dtype), B, heads, Nq, Nk, dh, dq.data_ptr(), _dt(dq.dtype),
                                       dk.data_ptr(), dv.data_ptr(), dk_bs, _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream())
        _check("ptdit_attn_bwd_tokens", st)
        return dq, dk, dv
    st = lib.ptdit_attn_bwd(q.data_ptr(), q_bs, k.data_ptr(), v.data_ptr(), kv_bs, _ptr(d_o), _dt(q.dtype),
                            B, heads, Nq, Nk, dh, dq.data_ptr(), dq_bs, dk.data_ptr(), dv.data_ptr(), dk_bs,
                            _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check("ptdit_attn_bwd", st)
    return dq, dk, dv


def proxy_pool_bwd(d_proxies: torch.Tensor, grid: Sequence[int], p: Sequence[int],
                   d_x: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """Backward of the window average: d_x[token] (+)= d_proxies[its proxy] / P (fp32)."""
    lib = load()
    B, F, H, W, D, _ = grid
    if _proxy_count(grid, p) is not None:
        _numel(d_proxies, _proxy_count(grid, p), "d_proxies")
    _numel(d_x, B * F * H * W * D, "d_x")
    if d_x is None:
        d_x = torch.empty(B, F * H * W, D, dtype=torch.float32, device=d_proxies.device)
    st = lib.ptdit_proxy_pool_bwd(_ptr(d_proxies), Grid(*grid), Win3(*p), _ptr(d_x), int(accumulate), _stream())
    _check("ptdit_proxy_pool_bwd", st)
    return d_x


def linear_bwd(x: torch.Tensor, w: torch.Tensor, d_y: torch.Tensor, want_dx: bool = True, want_dw: bool = True,
               want_db: bool = True, ws: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
               dw: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None,
               dx_add: Optional[torch.Tensor] = None, dx_bf16: Optional[torch.Tensor] = None):
    """Gradients of Y = X W^T + b: x [..., d_in], w [d_out, d_in] bf16, d_y [..., d_out].
    Returns fp32 (d_x or None, d_w or None, d_b or None): new tensors, or the
    given contiguous fp32 ones (e.g. row blocks of a larger gradient).
    dx_add (fp32, the shape of d_x; may be dx itself): added to d_x in the
    product's epilogue (ptdit_linear_bwd_ex). dx_bf16 (bf16): d_x rounded to
    bf16 as well; with want_dx False only the bf16 gradient is written."""
    lib = load()
    d_in, d_out = x.shape[-1], w.shape[0]
    rows = x.numel() // d_in
    if w.dtype != torch.bfloat16:
        raise ValueError("linear_bwd reads w as bf16 (the forward's weight dtype)")
    if tuple(w.shape) != (d_out, d_in):
        raise ValueError(f"w must be [d_out, {d_in}]")
    _numel(d_y, rows * d_out, "d_y")
    dev = x.device
    for t, n, name in ((dx, rows * d_in, "dx"), (dw, d_out * d_in, "dw"), (db, d_out, "db"),
                       (dx_add, rows * d_in, "dx_add")):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be fp32")
        _numel(t, n, name)
    if dx_bf16 is not None:
        if dx_bf16.dtype != torch.bfloat16:
            raise ValueError("dx_bf16 must be bf16")
        _numel(dx_bf16, rows * d_in, "dx_bf16")
    if dx_add is not None and not want_dx:
        raise ValueError("dx_add needs the fp32 d_x (want_dx)")
    if dx is None and want_dx:
        dx = torch.empty(*x.shape[:-1], d_in, dtype=torch.float32, device=dev)
    if dw is None and want_dw:
        dw = torch.empty(d_out, d_in, dtype=torch.float32, device=dev)
    if db is None and want_db:
        db = torch.empty(d_out, dtype=torch.float32, device=dev)
    need = int(lib.ptdit_linear_bwd_workspace_bytes(rows, d_in, d_out))
    ws = _ws(need, ws, dev)
    if dx_add is None and dx_bf16 is None:
        st = lib.ptdit_linear_bwd(_ptr(x), _dt(x.dtype), rows, d_in, d_out, _ptr(w), _ptr(d_y), _dt(d_y.dtype),
                                  _ptr(dx), _ptr(dw), _ptr(db), _ptr(ws), ws.numel() * ws.element_size(), _stream())
        _check("ptdit_linear_bwd", st)
    else:
        st = lib.ptdit_linear_bwd_ex(_ptr(x), _dt(x.dtype), rows, d_in, d_out, _ptr(w), _ptr(d_y), _dt(d_y.dtype),
                                     _ptr(dx), _ptr(dx_add), _ptr(dx_bf16), _ptr(dw), _ptr(db), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream())
        _check("ptdit_linear_bwd_ex", st)
    return dx, dw, db


MAX_DW_GROUP = 4   # PTDIT_MAX_DW_GROUP


def linear_bwd_dw_group(xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor],
                        dws: Optional[Sequence[torch.Tensor]] = None, dbs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                        want_db: bool = True, ws: Optional[torch.Tensor] = None):
    """Weight (and bias) gradients of up to MAX_DW_GROUP projections of one
    shape in one launch (ptdit_linear_bwd_dw_group): xs[i] [rows, d_in],
    dys[i] [rows, d_out], bf16 token-major. Returns (dws, dbs), fp32: the
    given tensors or new ones (dbs entries None without want_db)."""
    lib = load()
    n = len(xs)
    if n < 1 or n > MAX_DW_GROUP or len(dys) != n:
        raise ValueError(f"1..{MAX_DW_GROUP} products, as many dY as X")
    d_in, d_out = xs[0].shape[-1], dys[0].shape[-1]
    rows = xs[0].numel() // d_in
    for x, dy in zip(xs, dys):
        if x.dtype != torch.bfloat16 or dy.dtype != torch.bfloat16:
            raise ValueError("X and dY are bf16")
        _numel(x, rows * d_in, "x")
        _numel(dy, rows * d_out, "d_y")
    dev = xs[0].device
    if dws is None:
        dws = [torch.empty(d_out, d_in, dtype=torch.float32, device=dev) for _ in range(n)]
    if dbs is None:
        dbs = [torch.empty(d_out, dtype=torch.float32, device=dev) if want_db else None for _ in range(n)]
    for t, cnt, name in [(t, d_out * d_in, "dw") for t in dws] + [(t, d_out, "db") for t in dbs]:
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be fp32")
        _numel(t, cnt, name)
    need = int(lib.ptdit_linear_bwd_dw_group_workspace_bytes(n, rows, d_in, d_out))
    if need == 0:
        raise ValueError("shape outside the grouped weight gradient (rows % 32, 256 <= rows, 1024 <= d_out <= 4096)")
    ws = _ws(need, ws, dev)
    arr = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])
    st = lib.ptdit_linear_bwd_dw_group(n, arr(xs), arr(dys), rows, d_in, d_out, arr(dws), arr(dbs), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream())
    _check("ptdit_linear_bwd_dw_group", st)
    return dws, dbs


def trace_enable(kernel_class: int, capacity: int) -> None:
    _check("ptdit_trace_enable", load().ptdit_trace_enable(kernel_class, capacity))


def trace_read(max_n: int) -> list:
    buf = (ctypes.c_float * max_n)()
    n = load().ptdit_trace_read(buf, max_n)
    return [buf[i] for i in range(n)]


def trace_disable() -> None:
    load().ptdit_trace_disable()


# ----------------------------------------------------------------------------- recompute / chaining

def linear_heads(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], B: int, Ntok: int, heads: int,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B*Ntok, D] -> y = x W^T + b head-major [B, G, heads, Ntok, D/heads] (G = rows(w) / D)."""
    lib = load()
    D = x.shape[-1]
    if w.shape[1] != D or w.shape[0] % D:
        raise ValueError(f"w must be [G*{D}, {D}]")
    G = w.shape[0] // D
    _numel(x, B * Ntok * D, "x")
    _numel(b, G * D, "b")
    _numel(out, B * Ntok * G * D, "out")
    if out is None:
        out = torch.empty(B, G, heads, Ntok, D // heads, dtype=w.dtype, device=x.device)
    st = lib.ptdit_linear_heads(_ptr(x), _dt(x.dtype), B, Ntok, D, G, heads, _ptr(w), _ptr(b), _ptr(out),
                                _dt(w.dtype), _stream())
    _check("ptdit_linear_heads", st)
    return out


def window_attn(qkv: torch.Tensor, b_qkv: Optional[torch.Tensor], grid: Sequence[int], win: Sequence[int],
                shift: Sequence[int] = (0, 0, 0), out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Window / shifted-window attention core on head-major qkv [B, 3, heads, N, dh] -> O [B, N, D]."""
    lib = load()
    B, F, H, W, D, heads = grid
    N = F * H * W
    _numel(qkv, B * 3 * N * D, "qkv")
    _numel(b_qkv, 3 * D, "b_qkv")
    _numel(out, B * N * D, "out")
    if out is None:
        out = torch.empty(B, N, D, dtype=qkv.dtype, device=qkv.device)
    st = lib.ptdit_window_attn(_ptr(qkv), _ptr(b_qkv), _dt(qkv.dtype), Grid(*grid), Win3(*win), Win3(*shift),
                               _ptr(out), _stream())
    _check("ptdit_window_attn", st)
    return out


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Unmasked attention core: q [B, heads, Nq, dh], k / v [B, heads, Nk, dh] (views into
    fused buffers allowed) -> O [B, Nq, heads*dh]."""
    lib = load()
    B, heads, Nq, dh = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, heads, Nk, dh) or tuple(v.shape) != tuple(k.shape) or k.stride(0) != v.stride(0):
        raise ValueError("k and v must both be [B, heads, Nk, dh] with one batch stride")
    if len({q.dtype, k.dtype, v.dtype}) != 1:
        raise ValueError("q, k and v must share one dtype")
    q_bs, kv_bs = _bhld(q, "q"), _bhld(k, "k")
    _bhld(v, "v")
    _numel(out, B * Nq * heads * dh, "out")
    if out is None:
        out = torch.empty(B, Nq, heads * dh, dtype=q.dtype, device=q.device)
    need = int(lib.ptdit_attn_workspace_bytes(B, heads, Nk, _dt(q.dtype)))
    ws = _ws(need, ws, q.device) if need else None
    st = lib.ptdit_attn(q.data_ptr(), q_bs, k.data_ptr(), v.data_ptr(), kv_bs, _dt(q.dtype), B, heads, Nq, Nk, dh,
                        _ptr(out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("ptdit_attn", st)
    return out


def heads_to_tokens(src: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 [B, G, heads, Ntok, dh] -> [B, Ntok, G*heads*dh]."""
    lib = load()
    B, G, heads, Ntok, dh = src.shape
    if src.dtype != torch.float32:
        raise ValueError("heads_to_tokens moves fp32 gradients")
    _numel(out, src.numel(), "out")
    if out is None:
        out = torch.empty(B, Ntok, G * heads * dh, dtype=torch.float32, device=src.device)
    _check("ptdit_heads_to_tokens",
           lib.ptdit_heads_to_tokens(_ptr(src), B, G, heads, Ntok, dh, _ptr(out), _stream()))
    return out


def f32_to_bf16(src: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    if src.dtype != torch.float32:
        raise ValueError("f32_to_bf16 reads fp32")
    _numel(out, src.numel(), "out")
    if out is None:
        out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    _check("ptdit_f32_to_bf16", lib.ptdit_f32_to_bf16(_ptr(src), src.numel(), _ptr(out), _stream()))
    return out


def add_f32(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = a + b (fp32, element-wise; out may be a or b)."""
    lib = load()
    if a.dtype != torch.float32 or b.dtype != torch.float32:
        raise ValueError("add_f32 adds fp32 tensors")
    _numel(b, a.numel(), "b")
    _numel(out, a.numel(), "out")
    if out is None:
        out = torch.empty_like(a)
    _check("ptdit_add_f32", lib.ptdit_add_f32(_ptr(a), _ptr(b), a.numel(), _ptr(out), _stream()))
    return out


def calibrate_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """dst <- src byte for byte with the library's plain copy kernel (the
    known-size reference for hardware byte counters)."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("calibrate_copy takes contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("calibrate_copy: src and dst sizes differ")
    _check("ptdit_calibrate_copy", load().ptdit_calibrate_copy(_ptr(src), _ptr(dst), nbytes, _stream()))
    return dst


def calibrate(reps: int = 5) -> dict:
    """On-box ceilings: the sustained bf16 MFMA rate (back-to-back MFMAs on
    register operands over 1024 workgroups) and the streaming HBM read rate
    of a 2 GiB buffer (beyond the 256 MB last-level cache) and of a 38 MB
    one (the pooling kernel's size), each the best of `reps` event-timed runs
    (the 38 MB one also over workgroup counts). The 38 MB reads rotate over
    16 buffers written beforehand in the same order (613 MB in all), so each
    timed read finds its buffer mapped but evicted from the last-level cache."""
    lib = load()
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    flop = ctypes.c_int64(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    ms = best(lambda: _check("ptdit_calibrate_mfma",
                             lib.ptdit_calibrate_mfma(1024, 20000, _ptr(out), ctypes.byref(flop), _stream())))
    res = {"mfma_bf16_tflops": round(flop.value / (ms * 1e-3) / 1e12, 1)}
    for name, nbytes, grids in (("hbm_read_gbs", 2 << 30, (2048,)), ("hbm_read_gbs_38mb", 38_338_560, (512, 1024, 2048))):
        bufs = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(1 if nbytes > (1 << 30) else 16)]
        it = iter(range(1 << 30))
        ms = min(best(lambda: _check("ptdit_calibrate_read",
                                     lib.ptdit_calibrate_read(_ptr(bufs[next(it) % len(bufs)]), nbytes, nb, _ptr(out),
                                                              _stream())))
                 for nb in grids)
        res[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        del bufs
    return res
