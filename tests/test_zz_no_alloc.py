"""GPU test of ptdit_proxy_sa_noalloc, the entry point that allocates nothing
(its workspace is the library's static scratch): through the C ABI, two calls
in a row (the second smaller) against ptdit_proxy_sa with a workspace of its
own (same kernels, so bit-identical) and against the float64 oracle
(max-abs 2e-2, rel-L2 1e-2); and the host-side refusal of a problem larger
than the scratch. Collected last (test_zz_*), so a failure here hides no
other test."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import announce, assert_close, dev, host
from synth_inputs import WORKLOADS, make_all_weights, round_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_attention_pt_amd as P
    P.load()
    return P


def _proxies(B, M, D, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal((B, M, D)).astype(np.float32)


def test_noalloc_proxy_sa_matches_workspace_call_twice(P):
    from diffusion_transformer_attention_pt_amd import _lib
    wl = WORKLOADS["img2048"]
    ws_np = make_all_weights(wl)[0]                 # the proxy self-attention's weights
    w = _lib.AttnWeights.from_dict(ws_np, torch.bfloat16, "cuda")
    D, heads = wl.D, wl.heads
    # first call: the video's 864 proxies (bf16); then two batches of the
    # 2048^2 block's 256 proxies (fp32 stream, as in the block); then a
    # smaller problem, 1 x 100 bf16 proxies (each call smaller than the last)
    for (B, M, pdt), seed in (((1, 864, torch.bfloat16), 70), ((2, 256, torch.float32), 71),
                              ((1, 100, torch.bfloat16), 72)):
        announce(f"proxy_sa_noalloc B={B} M={M} {pdt}")
        x = _proxies(B, M, D, seed)
        if pdt == torch.bfloat16:
            x = round_bf16(x)
        xd = dev(x, pdt)
        out_na = torch.empty(B, M, D, dtype=torch.float32, device="cuda")
        out_ws = torch.empty_like(out_na)
        _lib.proxy_sa_noalloc(xd, heads, w, out_na, residual=True)
        _lib.proxy_sa(xd, heads, w, residual=True, out=out_ws)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), "no-allocation call differs from the workspace call"
        ref = O.proxy_sa(x.astype(np.float64), ws_np, heads, residual=True)
        assert_close(host(out_na) - x, ref - x, f"branch B={B} M={M}")


def test_noalloc_rejects_problems_beyond_the_scratch(P):
    from diffusion_transformer_attention_pt_amd import _lib
    wl = WORKLOADS["img2048"]
    w = _lib.AttnWeights.from_dict(make_all_weights(wl)[0], torch.bfloat16, "cuda")
    x = torch.zeros(1, 3641, wl.D, dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 3641, wl.D), 7.0, device="cuda")
    with pytest.raises(_lib.PtditError) as e:
        _lib.proxy_sa_noalloc(x, wl.heads, w, out)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call must leave its output untouched"
