"""PT-DiT attention core (Qihoo-T2X GIIM + TCM) on AMD MI355X (gfx950).

The compute path is libptdit.so: hand-written HIP kernels behind the C ABI
declared in include/ptdit.h. This package is a thin ctypes binding (_lib)
plus the five-call block composer (block). Importing it does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from ._lib import (AttnWeights, MlpWeights, PtditError, attn_bwd, linear, linear_bwd, load, mlp, proxy_pool,
                   proxy_pool_bwd,
                   proxy_sa, proxy_select, proxy_xattn, roll3d, shift_window_sa, version, window_attn_bwd, window_sa,
                   workspace_bytes)
from .block import PTBlockAttention

__all__ = ["AttnWeights", "MlpWeights", "PtditError", "PTBlockAttention", "attn_bwd", "linear", "linear_bwd", "load",
           "mlp",
           "proxy_pool", "proxy_pool_bwd", "proxy_sa", "proxy_select", "proxy_xattn", "roll3d", "shift_window_sa",
           "version", "window_attn_bwd", "window_sa", "workspace_bytes"]
