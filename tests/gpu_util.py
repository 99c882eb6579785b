"""Helpers for the GPU parity tests (device transfer, the tolerance bar)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerance for floating-point results (bf16 inputs, fp32 accumulation)
# against the float64 oracle: max-abs error 2e-2 and relative L2 error 1e-2.
ATOL = 2e-2
REL_L2 = 1e-2


def dev(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Host float32 values -> device tensor of `dtype`. bf16 inputs are already
    bf16-representable, so the cast is exact."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0
    return mx, rel


def assert_close(got, ref, what: str, atol: float = ATOL, rel_l2: float = REL_L2):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, rel = errors(got, ref)
    print(f"  {what}: max-abs {mx:.3e}  rel-L2 {rel:.3e}", flush=True)
    assert mx <= atol, f"{what}: max-abs {mx:.3e} > {atol}"
    assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e} > {rel_l2}"


def grad_bar(ref) -> float:
    """Max-abs bar of a gradient: 2e-2 scaled by the reference's largest
    magnitude when that exceeds 1 (a relative L-infinity bar). A gradient sums
    many products whose bf16 operands each carry a relative rounding of 2^-9,
    so its error grows with the size of its elements (dW, db and dK/dV sum
    over thousands of rows, and weight gradients are heavy-tailed: the largest
    element of the output projection's dW is about 7 times its RMS); for
    gradients of unit scale the bar is the forward's 2e-2. The relative-L2
    bar stays 1e-2."""
    ref = np.asarray(ref, np.float64)
    big = float(np.abs(ref).max()) if ref.size else 0.0
    return ATOL * max(1.0, big)


def assert_grad_close(got, ref, what: str):
    assert_close(got, ref, what, atol=grad_bar(ref), rel_l2=REL_L2)


def announce(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()
