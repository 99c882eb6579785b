"""PT-DiT attention core (Qihoo-T2X GIIM + TCM) on AMD MI355X (gfx950).

The compute path is libptdit.so: hand-written HIP kernels behind the C ABI
declared in include/ptdit.h. This package is a thin ctypes binding (_lib),
the five-call block composer (block) and its backward chain (block_bwd).
Importing it does not load the library; the first call does, and fails
loudly if it has not been built.
"""
from ._lib import (AttnWeights, MlpWeights, PtditError, add_f32, attn, attn_bwd, f32_to_bf16, heads_to_tokens, linear,
                   linear_bwd, linear_heads, load, mlp, proxy_pool, proxy_pool_bwd, proxy_sa, proxy_sa_noalloc,
                   proxy_select, proxy_xattn, roll3d, shift_window_sa, version, window_attn, window_attn_bwd,
                   window_sa, workspace_bytes)
from .block import PTBlockAttention
from .block_bwd import PTBlockBackward

__all__ = ["AttnWeights", "MlpWeights", "PtditError", "PTBlockAttention", "PTBlockBackward", "add_f32", "attn",
           "attn_bwd", "f32_to_bf16", "heads_to_tokens", "linear", "linear_bwd", "linear_heads", "load", "mlp",
           "proxy_pool", "proxy_pool_bwd", "proxy_sa", "proxy_sa_noalloc", "proxy_select", "proxy_xattn", "roll3d",
           "shift_window_sa", "version", "window_attn", "window_attn_bwd", "window_sa", "workspace_bytes"]
