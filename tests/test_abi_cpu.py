"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.
No kernel runs here (the calls below fail validation first)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from synth_inputs import ALL_WORKLOADS, WORKLOADS, WORKLOAD_ORDER

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ptdit.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ptdit_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from diffusion_transformer_attention_pt_amd import _lib
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    from diffusion_transformer_attention_pt_amd import _lib
    assert sorted(_lib.EXPORTED) == names


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.ptdit_version()
    for code in range(-9, 1):
        s = lib.ptdit_status_str(code)
        assert s and s != b"unknown status"
    assert lib.ptdit_status_str(-99) == b"unknown status"


def test_workspace_bytes(lib):
    from diffusion_transformer_attention_pt_amd._lib import Grid, Win3, OP_WINDOW_SA, OP_PROXY_XATTN, OP_PROXY_SA
    g = Grid(1, 1, 128, 128, 1152, 16)
    n = lib.ptdit_workspace_bytes(OP_WINDOW_SA, g, 0, Win3(1, 8, 8), 0)
    assert n == 4 * 16384 * 1152 * 2 + 3 * 1152 * 1152 * 2   # Q/K/V, O, packed w_qkv (bf16)
    assert lib.ptdit_workspace_bytes(OP_WINDOW_SA, g, 0, Win3(1, 8, 8), 1) == 4 * 16384 * 1152 * 4
    n = lib.ptdit_workspace_bytes(OP_PROXY_XATTN, g, 256, Win3(1, 1, 1), 1)
    assert n == (2 * 16384 * 1152 + 2 * 256 * 1152) * 4
    n = lib.ptdit_workspace_bytes(OP_PROXY_SA, Grid(2, 1, 1, 256, 1152, 16), 256, Win3(1, 1, 1), 0)
    assert n == 2 * 4 * 256 * 1152 * 2
    assert lib.ptdit_workspace_bytes(OP_WINDOW_SA, g, 0, Win3(1, 8, 8), 7) == 0


def test_host_validation_rejects_before_launch(lib):
    from diffusion_transformer_attention_pt_amd._lib import AttnW, Grid, Win3
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    g = Grid(1, 1, 16, 16, 1152, 16)
    # pool: window does not divide the grid
    assert lib.ptdit_proxy_pool(fake, 0, g, Win3(1, 3, 3), fake, 0, None) == -3
    # pool: null pointer
    assert lib.ptdit_proxy_pool(None, 0, g, Win3(1, 2, 2), fake, 0, None) == -1
    # pool: misaligned
    assert lib.ptdit_proxy_pool(ctypes.c_void_p((1 << 20) + 2), 0, g, Win3(1, 2, 2), fake, 0, None) == -5
    # pool: bad dtype, bad D
    assert lib.ptdit_proxy_pool(fake, 5, g, Win3(1, 2, 2), fake, 0, None) == -4
    assert lib.ptdit_proxy_pool(fake, 0, Grid(1, 1, 16, 16, 1150, 16), Win3(1, 2, 2), fake, 0, None) == -2
    w = AttnW(fake.value, None, fake.value, None)
    # window: head width without kernels, shift >= window, too-large window
    assert lib.ptdit_window_sa(fake, None, 0, Grid(1, 1, 16, 16, 1152, 12), Win3(1, 8, 8), ctypes.byref(w),
                               1, fake, None, 0, fake, 1 << 30, 0, None) == -2
    assert lib.ptdit_shift_window_sa(fake, None, 0, g, Win3(1, 8, 8), Win3(0, 8, 4), ctypes.byref(w), 1,
                                     fake, None, 0, fake, 1 << 30, 0, None) == -2
    assert lib.ptdit_window_sa(fake, None, 0, g, Win3(2, 8, 9), ctypes.byref(w), 1, fake, None, 0, fake,
                               1 << 30, 0, None) == -2
    # window: workspace too small
    far = ctypes.c_void_p(1 << 40)
    assert lib.ptdit_window_sa(fake, None, 0, g, Win3(1, 8, 8), ctypes.byref(w), 1, far, None, 0,
                               fake, 16, 0, None) == -6
    # window: output aliases the input
    assert lib.ptdit_window_sa(fake, None, 0, g, Win3(1, 8, 8), ctypes.byref(w), 1, fake, None, 0,
                               far, 1 << 30, 0, None) == -8
    # fp32 precision with bf16 activations
    assert lib.ptdit_window_sa(fake, None, 0, g, Win3(1, 8, 8), ctypes.byref(w), 1, fake, None, 0, fake,
                               1 << 30, 1, None) == -4
    # bf16 copies: only beside fp32 tensors, only with bf16 precision, aligned, not aliased
    x32, o32 = ctypes.c_void_p(1 << 41), ctypes.c_void_p(1 << 42)
    lo, ws = ctypes.c_void_p(1 << 43), ctypes.c_void_p(1 << 44)
    ok_args = dict(x=x32, xl=lo, xdt=1, out=o32, ol=None, odt=1, prec=0)

    def win(**kw):
        a = {**ok_args, **kw}
        return lib.ptdit_window_sa(a["x"], a["xl"], a["xdt"], g, Win3(1, 8, 8), ctypes.byref(w), 1, a["out"],
                                   a["ol"], a["odt"], ws, 1 << 30, a["prec"], None)
    assert win(xdt=0) == -4                                   # x_lowp beside a bf16 x
    assert win(xl=None, ol=lo, odt=0) == -4                   # out_lowp beside a bf16 out
    assert win(xl=None, ol=lo, prec=1) == -4                  # fp32 precision
    assert win(xl=ctypes.c_void_p((1 << 43) + 8)) == -5       # misaligned
    assert win(xl=None, ol=ctypes.c_void_p((1 << 41) + 4096)) == -8   # out_lowp inside x
    assert win(ol=lo) == -8                                   # out_lowp is x_lowp
    assert win(xl=ctypes.c_void_p((1 << 42) + 4096)) == -8    # out inside x_lowp's range
    assert lib.ptdit_proxy_xattn(x32, None, 1, g, fake, 0, 256, ctypes.byref(w), 1, o32, ctypes.c_void_p(1 << 44),
                                 1, ctypes.c_void_p(1 << 44), 1 << 30, 0, None) == -8  # out_lowp is the ws
    assert lib.ptdit_proxy_xattn(x32, None, 1, g, fake, 0, 256, ctypes.byref(w), 1, o32, lo, 0, ws, 1 << 30, 0,
                                 None) == -4                 # out_lowp beside a bf16 out
    assert lib.ptdit_proxy_xattn(fake, lo, 0, g, fake, 0, 256, ctypes.byref(w), 1, o32, None, 1, ws, 1 << 30, 0,
                                 None) == -4                 # x_lowp beside a bf16 x
    assert lib.ptdit_proxy_xattn(x32, ctypes.c_void_p((1 << 43) + 8), 1, g, fake, 0, 256, ctypes.byref(w), 1,
                                 o32, None, 1, ws, 1 << 30, 0, None) == -5   # misaligned x_lowp
    assert lib.ptdit_proxy_xattn(x32, lo, 1, g, fake, 0, 256, ctypes.byref(w), 1, o32, lo, 1, ws, 1 << 30, 0,
                                 None) == -8                 # out_lowp is x_lowp
    # inputs inside the workspace (the first projection writes it before the
    # last one reads the input as its residual)
    big = ctypes.c_void_p(1 << 45)
    inws = ctypes.c_void_p((1 << 45) + 4096)
    assert lib.ptdit_window_sa(inws, None, 0, g, Win3(1, 8, 8), ctypes.byref(w), 1, o32, None, 0, big, 1 << 30, 0,
                               None) == -8                   # x inside ws
    assert lib.ptdit_window_sa(x32, inws, 1, g, Win3(1, 8, 8), ctypes.byref(w), 1, o32, None, 1, big, 1 << 30, 0,
                               None) == -8                   # x_lowp inside ws
    assert lib.ptdit_proxy_xattn(inws, None, 0, g, fake, 0, 256, ctypes.byref(w), 1, o32, None, 0, big, 1 << 30, 0,
                                 None) == -8                 # x inside ws
    assert lib.ptdit_proxy_xattn(x32, inws, 1, g, fake, 0, 256, ctypes.byref(w), 1, o32, None, 1, big, 1 << 30, 0,
                                 None) == -8                 # x_lowp inside ws
    assert lib.ptdit_proxy_xattn(fake, None, 0, g, inws, 0, 256, ctypes.byref(w), 1, o32, None, 0, big, 1 << 30,
                                 0, None) == -8              # proxies inside ws
    assert lib.ptdit_proxy_sa(inws, 0, 1, 256, 1152, 16, ctypes.byref(w), 1, o32, 0, big, 1 << 30, 0,
                              None) == -8                    # proxies inside ws
    # no-allocation proxy SA: a problem beyond the static scratch is refused
    # on the host (3641 bf16 proxies of 1152 need more than 32 MiB)
    na = lambda B, M, prec=0: lib.ptdit_proxy_sa_noalloc(fake, prec, B, M, 1152, 16, ctypes.byref(w), 1, far,
                                                         prec, prec, None)
    assert na(1, 3641) == -9 and na(2, 1821) == -9 and na(1, 1821, prec=1) == -9
    assert na(0, 3641) == 0                                 # empty batch: nothing to do
    assert lib.ptdit_proxy_sa_noalloc(fake, 0, 1, 256, 1152, 12, ctypes.byref(w), 1, far, 0, 0, None) == -2
    # cross-attention with no proxies
    assert lib.ptdit_proxy_xattn(fake, None, 0, g, fake, 0, 0, ctypes.byref(w), 1, fake, None, 0, fake, 1 << 30, 0,
                                 None) == -2
    # null weights
    assert lib.ptdit_proxy_sa(fake, 0, 1, 256, 1152, 16, None, 1, fake, 0, fake, 1 << 30, 0, None) == -1
    # linear: d_in not a multiple of 8
    assert lib.ptdit_linear(fake, 0, 10, 12, 16, fake, None, None, 0, fake, 0, 0, None) == -2
    # selection: divisibility, dtype, D, nulls, alignment of the offsets, offsets inside the output
    sel = lib.ptdit_proxy_select
    assert sel(fake, 0, g, Win3(1, 3, 3), None, fake, 0, None) == -3
    assert sel(fake, 3, g, Win3(1, 2, 2), None, fake, 0, None) == -4
    assert sel(fake, 0, Grid(1, 1, 16, 16, 1150, 16), Win3(1, 2, 2), None, fake, 0, None) == -2
    assert sel(fake, 0, g, Win3(0, 2, 2), None, fake, 0, None) == -2
    assert sel(None, 0, g, Win3(1, 2, 2), None, fake, 0, None) == -1
    assert sel(fake, 0, g, Win3(1, 2, 2), ctypes.c_void_p((1 << 41) + 2), far, 0, None) == -5
    assert sel(fake, 0, g, Win3(1, 2, 2), ctypes.c_void_p((1 << 40) + 64), far, 0, None) == -8
    assert sel(None, 0, Grid(0, 1, 16, 16, 1152, 16), Win3(1, 2, 2), None, None, 0, None) == 0
    # MLP: widths, weights, dtypes, workspace, aliasing; zero rows is a no-op
    from diffusion_transformer_attention_pt_amd._lib import MlpW
    mw = MlpW(fake.value, None, fake.value, None)
    mlp = lambda x, rows, D, H, w, out, ws, wsb, prec=0, xl=None, xdt=0: lib.ptdit_mlp(
        x, xl, xdt, rows, D, H, w, 1, out, None, xdt, ws, wsb, prec, None)
    assert mlp(fake, 64, 1150, 4608, ctypes.byref(mw), far, far, 1 << 30) == -2
    assert mlp(fake, 64, 1152, 4604, ctypes.byref(mw), far, far, 1 << 30) == -2
    assert mlp(fake, 64, 1152, 4608, None, far, far, 1 << 30) == -1
    assert mlp(fake, 64, 1152, 4608, ctypes.byref(MlpW(fake.value, None, None, None)), far, far, 1 << 30) == -1
    assert mlp(fake, 64, 1152, 4608, ctypes.byref(mw), far, ctypes.c_void_p(1 << 41), 64) == -6
    assert mlp(fake, 64, 1152, 4608, ctypes.byref(mw), fake, ctypes.c_void_p(1 << 41), 1 << 30) == -8
    assert mlp(fake, 64, 1152, 4608, ctypes.byref(mw), far, ctypes.c_void_p(1 << 41), 1 << 30, prec=1) == -4
    assert mlp(fake, 64, 1152, 4608, ctypes.byref(mw), far, ctypes.c_void_p(1 << 41), 1 << 30,
               xl=ctypes.c_void_p(1 << 42)) == -4    # x_lowp beside a bf16 x
    assert mlp(ctypes.c_void_p((1 << 41) + 4096), 64, 1152, 4608, ctypes.byref(mw), far, ctypes.c_void_p(1 << 41),
               1 << 30) == -8                                # x inside ws
    assert mlp(x32, 64, 1152, 4608, ctypes.byref(mw), far, ctypes.c_void_p(1 << 44), 1 << 30, xdt=1,
               xl=ctypes.c_void_p((1 << 44) + 4096)) == -8   # x_lowp inside ws
    assert mlp(None, 0, 1152, 4608, ctypes.byref(mw), None, None, 0) == 0
    assert lib.ptdit_workspace_bytes(4, Grid(100, 1, 1, 1, 1152, 1), 4608, Win3(1, 1, 1), 0) >= 100 * 4608 * 2
    # roll: negative shift, D % 8, a grid row of 2^31 16-byte vectors (32-bit in-row index),
    # output inside the input
    roll = lib.ptdit_roll3d
    assert roll(fake, g, Win3(0, -1, 0), 0, far, 0, None) == -2
    assert roll(fake, Grid(1, 1, 16, 16, 1150, 16), Win3(0, 1, 1), 0, far, 0, None) == -2
    assert roll(fake, Grid(1, 1, 1, 1 << 20, 1 << 14, 16), Win3(0, 0, 1), 0, far, 0, None) == -2
    assert roll(fake, g, Win3(0, 1, 1), 0, ctypes.c_void_p((1 << 20) + 4096), 0, None) == -8
    # backward: window core (dtype, head width, window > 128, shift >= window, a padded grid
    # without d_b_kv, outputs over inputs)
    wb = lambda qkv, do, dt, gg, wn, sh, dq, db: lib.ptdit_window_attn_bwd(qkv, None, do, dt, gg, wn, sh, dq, db, None)
    gpad = Grid(1, 1, 20, 20, 1152, 16)
    d1, d2 = ctypes.c_void_p(1 << 41), ctypes.c_void_p(1 << 42)
    assert wb(fake, far, 3, g, Win3(1, 8, 8), Win3(0, 4, 4), d1, d2) == -4
    assert wb(fake, far, 0, Grid(1, 1, 16, 16, 1152, 12), Win3(1, 8, 8), Win3(0, 4, 4), d1, d2) == -2
    assert wb(fake, far, 0, g, Win3(3, 8, 8), Win3(0, 4, 4), d1, d2) == -2
    assert wb(fake, far, 0, g, Win3(1, 8, 8), Win3(0, 8, 4), d1, d2) == -2
    assert wb(fake, far, 0, gpad, Win3(1, 8, 8), Win3(0, 4, 4), d1, None) == -1
    assert wb(fake, far, 0, g, Win3(1, 8, 8), Win3(0, 4, 4), fake, d2) == -8
    assert wb(fake, far, 0, g, Win3(1, 8, 8), Win3(0, 4, 4), d1, ctypes.c_void_p((1 << 41) + 64)) == -8
    assert wb(None, None, 0, Grid(0, 1, 16, 16, 1152, 16), Win3(1, 8, 8), Win3(0, 4, 4), None, None) == 0
    # backward: dense core
    ab = lambda B, h, Nq, Nk, dh, qbs, kvbs, ws, wsb, dq=d1: lib.ptdit_attn_bwd(
        fake, qbs, far, far, kvbs, far, 0, B, h, Nq, Nk, dh, dq, h * Nq * dh, d2, ctypes.c_void_p(1 << 43),
        h * Nk * dh, ws, wsb, None)
    wsb = lib.ptdit_attn_bwd_workspace_bytes(1, 16, 2400, 150, 72)
    assert wsb >= 16 * 2400 * 3 * 4 + 3 * 16 * 150 * 2 * 72 * 4
    assert lib.ptdit_attn_bwd_workspace_bytes(1, 16, 256, 256, 80) == 0
    ws4 = ctypes.c_void_p(1 << 44)
    assert ab(1, 16, 2400, 150, 80, 16 * 2400 * 80, 16 * 150 * 80, ws4, wsb) == -2      # head width
    assert ab(300, 300, 64, 64, 72, 300 * 64 * 72, 300 * 64 * 72, ws4, 1 << 40) == -2   # B*heads
    assert ab(1, 16, 2400, 150, 72, 100, 16 * 150 * 72, ws4, wsb) == -2                 # q batch stride
    assert ab(1, 16, 2400, 0, 72, 16 * 2400 * 72, 0, ws4, wsb) == -2                    # no keys
    assert ab(1, 16, 2400, 150, 72, 16 * 2400 * 72, 16 * 150 * 72, ws4, 64) == -6       # workspace
    assert ab(1, 16, 2400, 150, 72, 16 * 2400 * 72, 16 * 150 * 72, ws4, wsb, dq=fake) == -8  # d_q over q
    assert ab(1, 16, 0, 150, 72, 0, 16 * 150 * 72, None, 0) == 0                        # no queries
    # backward: pooling
    pb = lib.ptdit_proxy_pool_bwd
    assert pb(fake, Grid(1, 1, 16, 16, 1150, 16), Win3(1, 4, 4), far, 0, None) == -2
    assert pb(fake, Grid(3, 1024, 1024, 1024, 8, 16), Win3(1, 4, 4), far, 0, None) == -2  # B*N > 2^31 - 1
    assert pb(fake, g, Win3(1, 3, 3), far, 0, None) == -3
    assert pb(None, g, Win3(1, 4, 4), far, 0, None) == -1
    assert pb(fake, g, Win3(1, 4, 4), ctypes.c_void_p((1 << 20) + 256), 0, None) == -8
    assert pb(None, Grid(0, 1, 16, 16, 1152, 16), Win3(1, 4, 4), None, 0, None) == 0
    # backward: projections (widths, nulls, workspace, aliasing, nothing wanted)
    lb = lambda x, rows, di, do_, w_, dy, dx, dw, db, ws, wsb: lib.ptdit_linear_bwd(
        x, 0, rows, di, do_, w_, dy, 1, dx, dw, db, ws, wsb, None)
    lws = lib.ptdit_linear_bwd_workspace_bytes(2400, 1152, 1152)
    assert lws >= 1152 * 1152 * 2 and lib.ptdit_linear_bwd_workspace_bytes(10, 12, 16) == 0
    o1, o2, o3, o4 = (ctypes.c_void_p(1 << k) for k in (41, 42, 43, 44))
    assert lb(fake, 2400, 1150, 1152, fake, far, o1, o2, o3, o4, lws) == -2
    assert lb(fake, 2400, 1152, 1152, fake, None, o1, o2, o3, o4, lws) == -1
    assert lb(None, 2400, 1152, 1152, fake, far, None, o2, None, o4, lws) == -1      # d_w needs x
    assert lb(fake, 2400, 1152, 1152, fake, far, o1, o2, o3, o4, 64) == -6
    assert lb(fake, 2400, 1152, 1152, fake, far, fake, o2, o3, o4, lws) == -8       # d_x over x
    assert lb(fake, 2400, 1152, 1152, fake, far, o1, o1, o3, o4, lws) == -8         # d_x over d_w
    assert lb(fake, 2400, 1152, 1152, fake, far, None, None, None, None, 0) == 0     # nothing wanted
    # empty inputs are a successful no-op
    assert lib.ptdit_proxy_pool(None, 0, Grid(0, 1, 16, 16, 1152, 16), Win3(1, 2, 2), None, 0, None) == 0
    assert lib.ptdit_window_sa(None, None, 0, Grid(0, 1, 16, 16, 1152, 16), Win3(1, 8, 8), ctypes.byref(w),
                               1, None, None, 0, None, 0, 0, None) == 0
    assert lib.ptdit_linear(None, 0, 0, 16, 16, None, None, None, 0, None, 0, 0, None) == 0


def test_block_flops_match_oracle_counters():
    """The FLOP figure the benchmark divides by equals the oracle's counters
    (projections over real rows; cores dense over windows, real queries)."""
    from diffusion_transformer_attention_pt_amd.block import PTBlockAttention
    for name in ALL_WORKLOADS:
        wl = WORKLOADS[name]
        blk = PTBlockAttention.__new__(PTBlockAttention)
        blk.B, (blk.F, blk.H, blk.W), blk.D, blk.N, blk.M, blk.win = wl.B, wl.grid, wl.D, wl.N, wl.M, wl.win
        f = blk.flops()
        pm = O.count_projection_macs(wl.grid, wl.p, wl.win, wl.D, B=wl.B)
        cm = O.count_core_macs(wl.grid, wl.p, wl.win, wl.D, B=wl.B, real_queries=True)
        assert f["projection"] == 2 * sum(pm.values())
        assert f["core"] == 2 * sum(cm.values())
    wl = WORKLOADS["img2048"]
    assert abs(PTBlockAttention.flops(_fake(wl))["total"] / 1e9 - 468.24) < 0.01


def _fake(wl):
    from diffusion_transformer_attention_pt_amd.block import PTBlockAttention
    blk = PTBlockAttention.__new__(PTBlockAttention)
    blk.B, (blk.F, blk.H, blk.W), blk.D, blk.N, blk.M, blk.win = wl.B, wl.grid, wl.D, wl.N, wl.M, wl.win
    return blk


def test_product_path_has_no_cpu_fallback():
    """The package must not import the oracle or compute on the CPU."""
    pkg = os.path.join(ROOT, "diffusion_transformer_attention_pt_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("oracle is", ""), fn
            assert "import numpy" not in src, fn


def test_binding_rejects_mismatched_shapes_before_any_call(lib):
    """The ctypes wrappers compare every tensor with the grid (and w's dtype
    for the projection gradients) and raise ValueError before the library is
    called, so a mismatch never reaches a kernel as an out-of-bounds index.
    CPU tensors suffice: the shape checks come before the device checks."""
    import torch
    from diffusion_transformer_attention_pt_amd import _lib as L

    D, heads = 64, 1
    grid = (1, 1, 8, 8, D, heads)
    x = torch.zeros(1, 64, D)
    short = torch.zeros(1, 63, D)
    w = L.AttnWeights(torch.zeros(3 * D, D), torch.zeros(3 * D), torch.zeros(D, D), torch.zeros(D))
    bad_w = L.AttnWeights(torch.zeros(2 * D, D), None, torch.zeros(D, D), None)
    cases = [
        lambda: L.proxy_pool(short, grid, (1, 2, 2)),
        lambda: L.proxy_pool(x, grid, (1, 2, 2), out=torch.zeros(1, 15, D)),
        lambda: L.proxy_select(short, grid, (1, 2, 2)),
        lambda: L.window_sa(short, grid, (1, 4, 4), w),
        lambda: L.window_sa(x, grid, (1, 4, 4), bad_w),
        lambda: L.window_sa(x, grid, (1, 4, 4), w, x_lowp=short),
        lambda: L.shift_window_sa(x, grid, (1, 4, 4), (0, 2, 2), w, out=short),
        lambda: L.proxy_xattn(short, grid, torch.zeros(1, 16, D), w),
        lambda: L.proxy_xattn(x, grid, torch.zeros(1, 16, D + 8), w),
        lambda: L.proxy_sa(torch.zeros(1, 16, D), heads, bad_w),
        lambda: L.roll3d(short, grid, (0, 1, 1)),
        lambda: L.window_attn_bwd(torch.zeros(1, 3, heads, 63, D), torch.zeros(1, 64, D), grid, (1, 4, 4)),
        lambda: L.window_attn_bwd(torch.zeros(1, 3, heads, 64, D), short, grid, (1, 4, 4)),
        lambda: L.attn_bwd(torch.zeros(1, 2, 10, 72), torch.zeros(1, 2, 5, 72), torch.zeros(1, 2, 6, 72),
                           torch.zeros(1, 10, 144)),
        lambda: L.attn_bwd(torch.zeros(1, 2, 10, 72), torch.zeros(1, 2, 5, 72), torch.zeros(1, 2, 5, 72),
                           torch.zeros(1, 9, 144)),
        lambda: L.proxy_pool_bwd(torch.zeros(1, 15, D), grid, (1, 2, 2)),
        lambda: L.linear_bwd(torch.zeros(4, D), torch.zeros(D, D), torch.zeros(4, D)),            # fp32 w
        lambda: L.linear_bwd(torch.zeros(4, D), torch.zeros(D, D, dtype=torch.bfloat16), torch.zeros(5, D)),
        lambda: L.linear(torch.zeros(4, D), torch.zeros(D, D + 8)),
    ]
    for i, f in enumerate(cases):
        with pytest.raises(ValueError):
            f()


def test_binding_leaves_divisibility_to_the_library(lib):
    """A proxy window that does not divide the grid is the library's error to
    report (PTDIT_ERR_DIVISIBILITY, checked on the host before any launch);
    the binding's shape checks do not pre-empt it."""
    import torch
    from diffusion_transformer_attention_pt_amd import _lib as L
    assert L._proxy_count((1, 1, 16, 16, 64, 1), (1, 5, 5)) is None
    assert L._proxy_count((2, 1, 16, 16, 64, 1), (1, 4, 4)) == 2 * 16 * 64


def test_chaining_calls_validate_on_the_host(lib):
    """Host checks of the recompute / chaining calls (nothing launched)."""
    import ctypes
    from diffusion_transformer_attention_pt_amd._lib import Grid, Win3
    a, b = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 34)
    assert lib.ptdit_add_f32(a, b, 6, a, None) == -2                          # n % 4
    assert lib.ptdit_add_f32(a, b, 64, ctypes.c_void_p((1 << 30) + 16), None) == -8   # shifted view of a
    assert lib.ptdit_add_f32(a, b, 64, ctypes.c_void_p((1 << 30) + 4), None) == -5    # misaligned
    assert lib.ptdit_add_f32(None, b, 64, a, None) == -1
    assert lib.ptdit_add_f32(a, b, 0, a, None) == 0
    assert lib.ptdit_f32_to_bf16(a, 12, b, None) == -2                        # n % 8
    assert lib.ptdit_f32_to_bf16(a, 64, ctypes.c_void_p((1 << 30) + 64), None) == -8
    assert lib.ptdit_heads_to_tokens(a, 1, 3, 16, 100, 70, b, None) == -2    # dh % 4
    assert lib.ptdit_heads_to_tokens(a, 1, 3, 16, 100, 72, a, None) == -8
    g = Grid(1, 1, 16, 16, 1152, 16)
    assert lib.ptdit_window_attn(a, None, 0, g, Win3(1, 8, 8), Win3(0, 8, 0), b, None) == -2   # shift >= window
    assert lib.ptdit_window_attn(a, None, 0, g, Win3(1, 16, 16), Win3(0, 0, 0), b, None) == -2  # 256 tokens
    assert lib.ptdit_window_attn(a, None, 0, g, Win3(1, 8, 8), Win3(0, 4, 4), a, None) == -8
    assert lib.ptdit_attn(a, 16 * 100 * 80, a, a, 16 * 50 * 80, 0, 1, 16, 100, 50, 80, b, None, 0, None) == -2
    assert lib.ptdit_attn(a, 16 * 100 * 72, a, a, 16 * 50 * 72, 0, 1, 16, 100, 0, 72, b, None, 0, None) == -2
    assert lib.ptdit_attn(a, 16 * 2048 * 72, a, a, 16 * 600 * 72, 0, 1, 16, 2048, 600, 72, b, None, 0, None) == -6
    assert lib.ptdit_attn_workspace_bytes(1, 16, 600, 0) > 0 and lib.ptdit_attn_workspace_bytes(1, 16, 600, 1) == 0
    assert lib.ptdit_linear_heads(a, 0, 1, 100, 1152, 4, 16, b, None, ctypes.c_void_p(1 << 38), 0, None) == -2
    assert lib.ptdit_linear_heads(a, 0, 1, 100, 1152, 3, 16, b, None, a, 0, None) == -8


def test_attn_bwd_alias_check_is_exact_for_interleaved_batches(lib):
    """d_q, d_k, d_v as interleaved views of one [B][3][heads][L][dh] fp32
    buffer (batch stride 3*heads*L*dh) are accepted for B > 1; a d_k view
    shifted by one element into d_q's block is refused (nothing launched:
    the workspace is too small, which is checked after the alias rule only
    when the rule passes)."""
    import ctypes
    B, heads, L, dh = 2, 16, 256, 72
    hk = heads * L * dh
    q = ctypes.c_void_p(1 << 30)
    kv = ctypes.c_void_p(1 << 32)
    base = 1 << 36
    args = lambda dq, dk, dv: lib.ptdit_attn_bwd(q, hk, kv, ctypes.c_void_p((1 << 32) + hk * 2), 2 * hk,
                                                 ctypes.c_void_p(1 << 34), 0, B, heads, L, L, dh,
                                                 ctypes.c_void_p(dq), 3 * hk, ctypes.c_void_p(dk),
                                                 ctypes.c_void_p(dv), 3 * hk, ctypes.c_void_p(1 << 40), 1 << 30,
                                                 None)
    # interleaved views: accepted by the alias rule; the call then needs a GPU,
    # so only the refusals are exercised here
    assert args(base, base + 4 * hk + 16, base + 8 * hk) == -8   # d_k overlaps d_v's block
    assert args(base, base + 4 * hk - 16, base + 8 * hk) == -8   # d_k overlaps d_q's block


def test_calibration_calls_validate_on_the_host(lib):
    """Host checks of the calibration calls (nothing launched)."""
    import ctypes
    a, b = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 34)
    assert lib.ptdit_calibrate_copy(a, b, 24, None) == -2                      # bytes % 16
    assert lib.ptdit_calibrate_copy(a, b, 0, None) == 0                        # nothing to copy
    assert lib.ptdit_calibrate_copy(None, b, 64, None) == -1
    assert lib.ptdit_calibrate_copy(ctypes.c_void_p((1 << 30) + 8), b, 64, None) == -5
    assert lib.ptdit_calibrate_copy(a, ctypes.c_void_p((1 << 30) + 32), 64, None) == -8   # overlap
    assert lib.ptdit_calibrate_read(a, 24, 64, b, None) == -2
    assert lib.ptdit_calibrate_read(a, 1 << 20, 64, ctypes.c_void_p((1 << 30) + 4096), None) == -8
    flop = ctypes.c_int64(0)
    assert lib.ptdit_calibrate_mfma(0, 10, b, ctypes.byref(flop), None) == -2
    assert lib.ptdit_calibrate_mfma(4, 10, None, ctypes.byref(flop), None) == -1


def test_linear_bwd_ex_validates_on_the_host(lib):
    """ptdit_linear_bwd_ex refusals (nothing launched)."""
    import ctypes
    x, w, dy = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 32), ctypes.c_void_p(1 << 34)
    dx, dw, db = ctypes.c_void_p(1 << 36), ctypes.c_void_p(1 << 38), ctypes.c_void_p(1 << 39)
    add, b16, ws = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 41), ctypes.c_void_p(1 << 42)
    rows, di, do = 256, 64, 128
    need = lib.ptdit_linear_bwd_workspace_bytes(rows, di, do)
    call = lambda dx_=dx, add_=add, b16_=b16, dw_=dw: lib.ptdit_linear_bwd_ex(
        x, 1, rows, di, do, w, dy, 1, dx_, add_, b16_, dw_, db, ws, need, None)
    assert call(dx_=None) == -1                                     # d_x_add needs the fp32 d_x
    assert call(b16_=ctypes.c_void_p((1 << 41) + 8)) == -5          # misaligned bf16 copy
    assert call(add_=ctypes.c_void_p((1 << 38) + 64)) == -8         # added gradient inside d_w
    assert call(b16_=ctypes.c_void_p((1 << 36) + 64)) == -8         # bf16 copy inside d_x
    assert call(add_=ctypes.c_void_p((1 << 36) + 16)) == -8         # a shifted view of d_x
    assert lib.ptdit_linear_bwd_ex(x, 1, 0, di, do, w, dy, 1, dx, add, b16, dw, db, ws, need, None) == 0


def test_keep_and_token_major_gradient_calls_validate_on_the_host(lib):
    """ptdit_window_sa_keep, ptdit_window_attn_bwd_tokens and
    ptdit_attn_bwd_tokens refusals (nothing launched): bf16 gradients only
    from bf16 inputs, the window call's own checks for the keep variant."""
    import ctypes
    from diffusion_transformer_attention_pt_amd._lib import AttnW, Grid, Win3
    fake = ctypes.c_void_p(1 << 20)
    g = Grid(1, 1, 16, 16, 1152, 16)
    w = AttnW(fake.value, None, fake.value, None)
    far, ws = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 44)
    # keep variant: same refusals as the window call
    assert lib.ptdit_window_sa_keep(None, None, 0, g, Win3(1, 8, 8), Win3(0, 0, 0), ctypes.byref(w), 1, far,
                                    None, 0, ws, 1 << 30, 0, None) == -1
    assert lib.ptdit_window_sa_keep(fake, None, 0, g, Win3(1, 8, 8), Win3(0, 8, 4), ctypes.byref(w), 1, far,
                                    None, 0, ws, 1 << 30, 0, None) == -2
    assert lib.ptdit_window_sa_keep(fake, None, 0, g, Win3(1, 8, 8), Win3(0, 4, 4), ctypes.byref(w), 1, far,
                                    None, 0, ws, 16, 0, None) == -6
    assert lib.ptdit_window_sa_keep(fake, None, 0, Grid(1, 1, 0, 16, 1152, 16), Win3(1, 8, 8), Win3(0, 4, 4),
                                    ctypes.byref(w), 1, far, None, 0, ws, 16, 0, None) == 0  # nothing to do
    # window gradients: bf16 output from fp32 inputs is refused, a bad dtype too
    qkv, do, dq = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 32), ctypes.c_void_p(1 << 34)
    assert lib.ptdit_window_attn_bwd_tokens(qkv, None, do, 1, g, Win3(1, 8, 8), Win3(0, 4, 4), dq, 0, None,
                                            None) == -4
    assert lib.ptdit_window_attn_bwd_tokens(qkv, None, do, 0, g, Win3(1, 8, 8), Win3(0, 4, 4), dq, 7, None,
                                            None) == -4
    assert lib.ptdit_window_attn_bwd_tokens(qkv, None, do, 0, g, Win3(1, 8, 8), Win3(0, 4, 4),
                                            ctypes.c_void_p((1 << 30) + 64), 0, None, None) == -8  # dq in qkv
    # dense gradients with token-major dQ: the same dtype rule, the alias check
    # against the token-major extent
    k, v, dk, dv = (ctypes.c_void_p(1 << s) for s in (36, 37, 38, 39))
    B, heads, Nq, Nk, dh = 1, 16, 1024, 256, 72
    need = lib.ptdit_attn_bwd_workspace_bytes(B, heads, Nq, Nk, dh)
    call = lambda dt, qdt, dq_=dq: lib.ptdit_attn_bwd_tokens(qkv, heads * Nq * dh, k, v, heads * Nk * dh, do, dt,
                                                             B, heads, Nq, Nk, dh, dq_, qdt, dk, dv,
                                                             heads * Nk * dh, ws, need, None)
    assert call(1, 0) == -4                                         # bf16 dQ from fp32 inputs
    assert call(0, 0, dq_=ctypes.c_void_p((1 << 32) + 1024)) == -8  # dQ inside d_o
    assert call(0, 0, dq_=ctypes.c_void_p((1 << 34) + 8)) == -5     # misaligned


def test_window_weight_packing_validates_on_the_host(lib):
    """ptdit_window_packed_bytes / ptdit_pack_window_weights: the size is
    3 D^2 bf16 where the fused kernel applies, 0 elsewhere; refusals before
    any launch (null, misaligned, unsupported shape, packed copy over w_qkv);
    a misaligned packed copy in ptdit_attn_w is refused by the window call."""
    import ctypes
    from diffusion_transformer_attention_pt_amd._lib import AttnW, Grid, Win3
    assert lib.ptdit_window_packed_bytes(1152, 16) == 3 * 1152 * 1152 * 2
    assert lib.ptdit_window_packed_bytes(2304, 32) == 3 * 2304 * 2304 * 2
    for D, heads in ((1024, 16), (576, 8), (1152, 0), (0, 16), (1152, 15), (1152, 12)):
        assert lib.ptdit_window_packed_bytes(D, heads) == 0, (D, heads)
    fake, far = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 40)
    assert lib.ptdit_pack_window_weights(None, 1152, 16, far, None) == -1
    assert lib.ptdit_pack_window_weights(fake, 1152, 16, None, None) == -1
    assert lib.ptdit_pack_window_weights(fake, 1152, 16, ctypes.c_void_p((1 << 40) + 8), None) == -5
    assert lib.ptdit_pack_window_weights(fake, 1024, 16, far, None) == -2
    assert lib.ptdit_pack_window_weights(fake, 1152, 16, ctypes.c_void_p((1 << 20) + 4096), None) == -8
    w = AttnW(fake.value, None, fake.value, None, (1 << 40) + 8)
    assert lib.ptdit_window_sa(fake, None, 0, Grid(1, 1, 16, 16, 1152, 16), Win3(1, 8, 8), ctypes.byref(w),
                               1, far, None, 0, ctypes.c_void_p(1 << 44), 1 << 30, 0, None) == -5


def test_grouped_weight_gradient_validates_on_the_host(lib):
    """ptdit_linear_bwd_dw_group refusals before any launch, and its
    workspace size (0 outside the shape rules)."""
    import ctypes
    vp = ctypes.c_void_p
    assert lib.ptdit_linear_bwd_dw_group_workspace_bytes(4, 16384, 1152, 1152) > 0
    for n, rows, di, do in ((0, 16384, 1152, 1152), (5, 16384, 1152, 1152), (2, 16400, 1152, 1152),
                            (2, 128, 1152, 1152), (2, 16384, 1152, 512), (2, 16384, 8192, 1152)):
        assert lib.ptdit_linear_bwd_dw_group_workspace_bytes(n, rows, di, do) == 0, (n, rows, di, do)
    base = 1 << 32
    arr = lambda *p: (vp * len(p))(*p)
    x, dy, dw = arr(base, base + (1 << 28)), arr(base + (2 << 28), base + (3 << 28)), arr(1 << 40, (1 << 40) + (1 << 24))
    ws, need = vp(1 << 44), lib.ptdit_linear_bwd_dw_group_workspace_bytes(2, 16384, 1152, 1152)
    call = lambda n=2, x_=x, dy_=dy, dw_=dw, db_=None, rows=16384, ws_=ws, nb=need: \
        lib.ptdit_linear_bwd_dw_group(n, x_, dy_, rows, 1152, 1152, dw_, db_, ws_, nb, None)
    assert call(n=5) == -2
    assert call(x_=None) == -1
    assert call(dw_=arr(1 << 40, None)) == -1
    assert call(rows=16400) == -2                      # not a multiple of 32
    assert call(nb=need - 1) == -6
    assert call(ws_=vp((1 << 44) + 4)) == -5
    assert call(dw_=arr(1 << 40, (1 << 40) + 8)) == -5  # misaligned second output
    assert call(dw_=arr(1 << 40, (1 << 40) + 4096)) == -8  # the outputs overlap
    assert call(dw_=arr(base + 64, 1 << 42)) == -8     # an output inside X_0
    assert call(rows=0) == 0
