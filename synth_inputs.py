"""Seeded synthetic inputs for the PT-DiT attention core (GIIM + TCM).

This module is shared by the CPU oracle, the GPU tests and the benchmark. It
only draws random numbers and names the workload shapes; it holds none of the
method's arithmetic (no pooling, no projection, no attention).

Workloads stand in for the image / video resolutions the Qihoo-T2X reading
note (page "Qihoo-T2X — Proxy-Tokenized DiT", section 3 "Method", compression
ratios paragraph) trains and samples at: only the latent token grid enters
the attention core, so no dataset or trained weight is needed.

Value recipe (stated once, used everywhere):
  * activations x ~ N(0, 1)
  * every projection weight and bias ~ N(0, 0.02); output projections are
    random too (not zero-initialised), otherwise the GIIM branch is zero
  * drawn in float32 with numpy.random.Generator(PCG64(seed));
    seed(x) = 1000*k, seed(attention a, tensor j) = 1000*k + 1 + 8*a + j,
    a in {0: proxy SA, 1: cross-attention, 2: WSA, 3: SWSA},
    j in {Wq, bq, Wk, bk, Wv, bv, Wo, bo}
  * bf16 workloads round every drawn value to bf16 (round-to-nearest-even)
    once, on the host; both the oracle and the GPU consume those values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

WEIGHT_NAMES = ("wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo")
ATTN_NAMES = ("proxy", "cross", "wsa", "swsa")


@dataclass(frozen=True)
class Workload:
    """One PT-block attention workload: token grid, proxy window, TCM window."""

    name: str
    index: int            # k: selects the seeds
    B: int
    F: int
    H: int
    W: int
    D: int
    heads: int
    p: Tuple[int, int, int]        # proxy (pooling) window (p_t, p_h, p_w)
    win: Tuple[int, int, int]      # TCM window (w_t, w_h, w_w)
    shift: Tuple[int, int, int]    # SWSA cyclic shift (s_t, s_h, s_w)
    dtype: str                     # "bf16" or "f32"
    note: str = ""

    @property
    def N(self) -> int:
        return self.F * self.H * self.W

    @property
    def M(self) -> int:
        return (self.F // self.p[0]) * (self.H // self.p[1]) * (self.W // self.p[2])

    @property
    def dh(self) -> int:
        return self.D // self.heads

    @property
    def grid(self) -> Tuple[int, int, int]:
        return (self.F, self.H, self.W)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads of this attention core. Index k selects the seeds.
WORKLOADS: Dict[str, Workload] = {
    "img256_f32": Workload("img256_f32", 1, B=1, F=1, H=32, W=32, D=1152, heads=16,
                           p=(1, 2, 2), win=(1, 8, 8), shift=(0, 4, 4), dtype="f32",
                           note="N=1024, 256 proxies, fp32"),
    "img1024": Workload("img1024", 2, B=2, F=1, H=64, W=64, D=1152, heads=16,
                        p=(1, 4, 4), win=(1, 8, 8), shift=(0, 4, 4), dtype="bf16",
                        note="N=4096 x batch 2, 256 proxies"),
    "img2048": Workload("img2048", 3, B=1, F=1, H=128, W=128, D=1152, heads=16,
                        p=(1, 8, 8), win=(1, 8, 8), shift=(0, 4, 4), dtype="bf16",
                        note="N=16384, 256 proxies (headline)"),
    "video16x30x45": Workload("video16x30x45", 4, B=1, F=16, H=30, W=45, D=1152, heads=16,
                              p=(1, 5, 5), win=(2, 8, 8), shift=(1, 4, 4), dtype="bf16",
                              note="N=21600, 864 proxies, grid zero-padded to 16x32x48 for TCM"),
    "img4096": Workload("img4096", 5, B=1, F=1, H=256, W=256, D=1152, heads=16,
                        p=(1, 16, 16), win=(1, 8, 8), shift=(0, 4, 4), dtype="bf16",
                        note="N=65536, 256 proxies"),
}
WORKLOAD_ORDER: List[str] = ["img256_f32", "img1024", "img2048", "video16x30x45", "img4096"]

# The pages' own video settings, beyond the five above. Video compresses time
# by p_f = 4 (Qihoo-T2X, section 3, compression ratios); the spatial ratio
# follows the image schedule for the view size (512 -> (4, 4)).
#  * the 16x30x45 video grid with p_f = 4: 4x6x9 = 216 proxies;
#  * multi-view generation read as a pseudo-video of 24 views, each a 512^2
#    image (32x32 latent tokens after 8x VAE and 2x2 patches): 24x32x32;
#  * long video, 512^2 x 288 frames, read as 72 latent frames (4x temporal
#    VAE) of 32x32 tokens: 73,728 tokens, 18x8x8 = 1152 proxies.
EXTRA_WORKLOADS: Dict[str, Workload] = {
    "video16x30x45_pf4": Workload("video16x30x45_pf4", 6, B=1, F=16, H=30, W=45, D=1152, heads=16,
                                  p=(4, 5, 5), win=(2, 8, 8), shift=(1, 4, 4), dtype="bf16",
                                  note="N=21600, p_f=4: 216 proxies, grid zero-padded to 16x32x48 for TCM"),
    "mview24x32x32": Workload("mview24x32x32", 8, B=1, F=24, H=32, W=32, D=1152, heads=16,
                              p=(4, 4, 4), win=(2, 8, 8), shift=(1, 4, 4), dtype="bf16",
                              note="N=24576 (24 views of 32x32), 384 proxies"),
    "video72x32x32": Workload("video72x32x32", 9, B=1, F=72, H=32, W=32, D=1152, heads=16,
                              p=(4, 4, 4), win=(2, 8, 8), shift=(1, 4, 4), dtype="bf16",
                              note="N=73728 (long video), 1152 proxies"),
}
WORKLOADS.update(EXTRA_WORKLOADS)
ALL_WORKLOADS: List[str] = WORKLOAD_ORDER + list(EXTRA_WORKLOADS)
HEADLINE = "img2048"


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Uses torch's float32 -> bfloat16 cast (round-to-nearest-even), so the
    rounding used to *make* bf16 inputs is a library routine, not code of
    either the oracle or the GPU path.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _normal(seed: int, shape, scale: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def make_x(wl: Workload, seed: int | None = None, scale: float = 1.0) -> np.ndarray:
    """Activations [B, N, D] (tokens row-major over (f, h, w)), float32 values."""
    s = 1000 * wl.index if seed is None else seed
    x = _normal(s, (wl.B, wl.N, wl.D), scale)
    return round_bf16(x) if wl.dtype == "bf16" else x


def make_weights(wl: Workload, attn: int, seed_base: int | None = None,
                 scale: float = 0.02) -> Dict[str, np.ndarray]:
    """Weights of attention `attn` (0 proxy SA, 1 cross, 2 WSA, 3 SWSA).

    W* are [D_out, D_in] (y = x W^T + b), b* are [D]. float32 values.
    """
    base = 1000 * wl.index if seed_base is None else seed_base
    out = {}
    D = wl.D
    for j, name in enumerate(WEIGHT_NAMES):
        shape = (D, D) if name.startswith("w") else (D,)
        v = _normal(base + 1 + 8 * attn + j, shape, scale)
        out[name] = round_bf16(v) if wl.dtype == "bf16" else v
    return out


TEXT_TOKENS = 120  # caption length of the text cross-attention


def make_text(wl: Workload, L: int = TEXT_TOKENS, seed: int | None = None) -> np.ndarray:
    """Caption embeddings [B, L, D] (already projected to D), N(0, 1)."""
    s = 1000 * wl.index + 997 if seed is None else seed
    t = _normal(s, (wl.B, L, wl.D), 1.0)
    return round_bf16(t) if wl.dtype == "bf16" else t


def make_mlp_weights(wl: Workload, hidden: int | None = None, seed_base: int | None = None,
                     scale: float = 0.02) -> Dict[str, np.ndarray]:
    """MLP weights: w1 [H, D], b1 [H], w2 [D, H], b2 [D], N(0, scale), H = 4D."""
    H = 4 * wl.D if hidden is None else hidden
    base = 1000 * wl.index + 60 if seed_base is None else seed_base
    shapes = {"w1": (H, wl.D), "b1": (H,), "w2": (wl.D, H), "b2": (wl.D,)}
    out = {}
    for j, (name, shape) in enumerate(shapes.items()):
        v = _normal(base + j, shape, scale)
        out[name] = round_bf16(v) if wl.dtype == "bf16" else v
    return out


def make_proxy_offsets(wl: Workload, seed: int | None = None) -> np.ndarray:
    """Window-local token offsets for random proxy extraction, int32 [B, M],
    uniform over the P = p_t*p_h*p_w tokens of each window (the draws the
    Random variant makes, passed to both sides as inputs)."""
    s = 1000 * wl.index + 999 if seed is None else seed
    g = np.random.Generator(np.random.PCG64(s))
    P = wl.p[0] * wl.p[1] * wl.p[2]
    return g.integers(0, P, size=(wl.B, wl.M), dtype=np.int32)


def make_all_weights(wl: Workload, **kw) -> List[Dict[str, np.ndarray]]:
    return [make_weights(wl, a, **kw) for a in range(4)]


def make_int_x(wl: Workload, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integer-valued activations in [lo, hi] (exact in bf16 and fp32)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(lo, hi + 1, size=(wl.B, wl.N, wl.D)).astype(np.float32)


def tiny(name: str = "tiny", *, B=1, F=1, H=8, W=8, D=16, heads=2, p=(1, 2, 2),
         win=(1, 4, 4), shift=(0, 2, 2), dtype="f32", index=90) -> Workload:
    """A small workload for brute-force pins and fast parity cases."""
    return Workload(name, index, B=B, F=F, H=H, W=W, D=D, heads=heads, p=p, win=win,
                    shift=shift, dtype=dtype)


def make_attn_grad_inputs(B: int, heads: int, Nq: int, Nk: int, dh: int, seed: int, scale: float = 1.0,
                          dtype: str = "bf16"):
    """Inputs of an attention-core backward: q [B, heads, Nq, dh], k, v
    [B, heads, Nk, dh] (standard normal times `scale` for q and k, so the
    scores q.k / sqrt(dh) have standard deviation scale^2), and the output
    gradient d_o [B, Nq, heads*dh] (standard normal). bf16-representable
    float32 when dtype is "bf16"."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, heads, Nq, dh), dtype=np.float32) * scale
    k = g.standard_normal((B, heads, Nk, dh), dtype=np.float32) * scale
    v = g.standard_normal((B, heads, Nk, dh), dtype=np.float32)
    do = g.standard_normal((B, Nq, heads * dh), dtype=np.float32)
    if dtype == "bf16":
        q, k, v, do = (round_bf16(a) for a in (q, k, v, do))
    return q, k, v, do
