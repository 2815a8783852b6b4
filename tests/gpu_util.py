"""Shared helpers of the GPU tests: seeded inputs, running the library and
the oracle on the same values, and element-wise comparison."""
import sys

import numpy as np
import torch

import conv1d_implicit_gemm_amd as c1g
import oracle
from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs, to_f64_numpy

DEV = "cuda:0"
TOL_F32 = 1e-4   # max-abs after normalisation, fp32 inputs
TOL_BF16 = 2e-2  # max-abs after normalisation, bf16 inputs


def announce(*what):
    """Name the case before any GPU work so a fault can be attributed."""
    print("[gpu-case]", *what, flush=True)
    sys.stdout.flush()


def to_dev(t):
    return None if t is None else t.to(DEV).contiguous()


def run_library(wl: Workload, inp: dict, *, return_stats=False, poison=True):
    """conv1d_gn_forward (or conv1d_forward when the workload has no norm
    and no epilogue) on device copies of the inputs."""
    x, w = to_dev(inp["x"]), to_dev(inp["w"])
    b, ga, be, b2 = (to_dev(inp[k]) for k in ("bias", "gamma", "beta", "bias2"))
    T_out = c1g.out_len(c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K, stride=wl.stride,
                                      dilation=wl.dilation, pad_left=wl.pad_left,
                                      pad_right=wl.pad_right))
    out = torch.full((wl.N, wl.C_out, T_out), float("nan") if poison else 0.0, device=DEV)
    if wl.norm is None and not wl.rowmin_bias:
        c1g.conv1d_forward(x, w, b, stride=wl.stride, dilation=wl.dilation,
                           pad_left=wl.pad_left, pad_right=wl.pad_right, out=out)
        res = (out, None, None)
    else:
        res = c1g.conv1d_gn_forward(x, w, b, stride=wl.stride, dilation=wl.dilation,
                                    pad_left=wl.pad_left, pad_right=wl.pad_right,
                                    norm=wl.norm, groups=wl.G, eps=wl.eps, gamma=ga, beta=be,
                                    rowmin_bias=b2, return_stats=True, out=out)
    torch.cuda.synchronize()
    return res if return_stats else res[0]


def run_oracle(wl: Workload, inp: dict, n_slice=None):
    """The oracle on the same (widened) values; n_slice restricts the batch."""
    f = to_f64_numpy
    x = f(inp["x"])
    if n_slice is not None:
        x = x[n_slice]
    return oracle.forward(x, f(inp["w"]), f(inp["bias"]), stride=wl.stride,
                          dilation=wl.dilation, pad_left=wl.pad_left, pad_right=wl.pad_right,
                          norm=wl.norm, G=wl.G, eps=wl.eps, gamma=f(inp["gamma"]),
                          beta=f(inp["beta"]), bias2=f(inp["bias2"]))


def max_abs_err(got, want):
    g = got.detach().to("cpu").to(torch.float64).numpy()
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.isfinite(g).all(), "non-finite output (unwritten element?)"
    return float(np.abs(g - want).max())


def tol_for(wl: Workload):
    return TOL_BF16 if wl.dtype == "bf16" else TOL_F32


def check_parity(wl: Workload, seed=0):
    announce(wl.name, wl, "seed", seed)
    inp = make_inputs(wl, seed)
    got, mean, rstd = run_library(wl, inp, return_stats=True)
    ref = run_oracle(wl, inp)
    err = max_abs_err(got, ref["out"])
    assert err <= tol_for(wl), "%s: max abs err %.3g > %.3g" % (wl.name, err, tol_for(wl))
    if mean is not None and ref["mean"] is not None:
        em = max_abs_err(mean, ref["mean"])
        er = float(np.max(np.abs(rstd.cpu().double().numpy() - ref["rstd"]) / ref["rstd"]))
        assert em <= 1e-4 * max(1.0, float(np.abs(ref["mean"]).max())), em
        assert er <= 1e-4, er
    return err
