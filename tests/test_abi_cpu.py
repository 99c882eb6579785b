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
    for code in range(-8, 1):
        s = lib.ptdit_status_str(code)
        assert s and s != b"unknown status"
    assert lib.ptdit_status_str(-99) == b"unknown status"


def test_workspace_bytes(lib):
    from diffusion_transformer_attention_pt_amd._lib import Grid, Win3, OP_WINDOW_SA, OP_PROXY_XATTN, OP_PROXY_SA
    g = Grid(1, 1, 128, 128, 1152, 16)
    n = lib.ptdit_workspace_bytes(OP_WINDOW_SA, g, 0, Win3(1, 8, 8), 0)
    assert n == 4 * 16384 * 1152 * 2
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
