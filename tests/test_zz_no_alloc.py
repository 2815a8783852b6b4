"""conv1d_gn_forward_noalloc, the entry point for callers that cannot
allocate (its workspace is the library's static device scratch), against
conv1d_gn_forward with a caller-allocated workspace: the same kernels, so the
same bits, on consecutive calls whose problems shrink (the scratch keeps the
previous call's contents), and within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import (DEV, announce, library_route, max_abs_err, run_library, run_oracle,
                            to_dev, tol_for)

pytestmark = pytest.mark.gpu

W = Workload
BF = dict(dtype="bf16")
# largest first: each later call runs on scratch the earlier ones left behind
SEQUENCE = [
    (W("noalloc_bf16_persist_gn", N=6, C_in=64, C_out=256, T=1100, K=5, dilation=2,
       pad_left=4, pad_right=4, G=16, **BF), "fused_persistent"),
    (W("noalloc_f32_split_ln", N=3, C_in=40, C_out=200, T=700, K=3, pad_left=1, pad_right=1,
       norm="layer_channels"), "split"),
    (W("noalloc_bf16_split_gn_rowmin", N=2, C_in=32, C_out=64, T=96, K=3, pad_left=1,
       pad_right=1, G=4, rowmin_bias=True, **BF), "split"),
    (W("noalloc_f32_fused_gn", N=2, C_in=16, C_out=32, T=256, K=3, pad_left=1, pad_right=1,
       G=8), "fused_single_pass"),
]


def _noalloc(wl, inp):
    x, w = to_dev(inp["x"]), to_dev(inp["w"])
    b, ga, be, b2 = (to_dev(inp[k]) for k in ("bias", "gamma", "beta", "bias2"))
    T_out = c1g.out_len(c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K, stride=wl.stride,
                                      dilation=wl.dilation, pad_left=wl.pad_left,
                                      pad_right=wl.pad_right))
    out = torch.full((wl.N, wl.C_out, T_out), float("nan"), device=DEV)
    shp = (wl.N, wl.G) if wl.norm == "group" else (wl.N, T_out)
    mean = torch.full(shp, float("nan"), device=DEV)
    rstd = torch.full(shp, float("nan"), device=DEV)
    c1g.conv1d_gn_forward_noalloc(x, w, b, out=out, stride=wl.stride, dilation=wl.dilation,
                                  pad_left=wl.pad_left, pad_right=wl.pad_right, norm=wl.norm,
                                  groups=wl.G, eps=wl.eps, gamma=ga, beta=be, rowmin_bias=b2,
                                  mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    return out, mean, rstd


def test_noalloc_matches_workspace_entry_point():
    sizes = []
    for wl, route in SEQUENCE:
        assert library_route(wl) == route
        need = c1g.conv1d_gn_workspace_size(
            c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K, stride=wl.stride,
                          dilation=wl.dilation, pad_left=wl.pad_left, pad_right=wl.pad_right,
                          dtype=c1g.C1G_BF16 if wl.dtype == "bf16" else c1g.C1G_F32),
            c1g.make_norm(wl.norm, wl.G, wl.eps, wl.rowmin_bias))
        assert need <= c1g.NOALLOC_SCRATCH_BYTES
        sizes.append(need)
        announce("noalloc", wl.name, route, "workspace", need)
        inp = make_inputs(wl, 9)
        ref_out, ref_mean, ref_rstd = run_library(wl, inp, return_stats=True)
        out, mean, rstd = _noalloc(wl, inp)
        assert torch.equal(out, ref_out), wl.name
        assert torch.equal(mean, ref_mean) and torch.equal(rstd, ref_rstd), wl.name
        ref = run_oracle(wl, inp)
        assert max_abs_err(out, ref["out"]) <= tol_for(wl), wl.name
        assert max_abs_err(mean, ref["mean"]) <= 1e-4, wl.name
        r = rstd.cpu().double().numpy()
        assert float(np.max(np.abs(r / ref["rstd"] - 1))) <= 1e-4, wl.name
    # each call needs less scratch than the one before (it runs on what is left)
    assert sizes == sorted(sizes, reverse=True)


def test_noalloc_repeat_after_larger_call():
    """The first problem again, after the smaller ones have overwritten the
    scratch: the same bits as its first run."""
    wl = SEQUENCE[0][0]
    announce("noalloc repeat", wl.name)
    inp = make_inputs(wl, 9)
    first = _noalloc(wl, inp)
    small = SEQUENCE[2][0]
    _noalloc(small, make_inputs(small, 1))
    again = _noalloc(wl, inp)
    for a, b in zip(first, again):
        assert torch.isfinite(a).all() and torch.equal(a, b)
