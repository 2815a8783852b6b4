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
# unit roundoff of bf16 (8 significant bits, round to nearest even): a bf16
# output adds at most BF16_U * |value| per rounding
BF16_U = 2.0 ** -8


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
    if wl.channels_last:  # the same values, laid out [N, T, C_in]
        x = x.transpose(1, 2).contiguous()
    b, ga, be, b2 = (to_dev(inp[k]) for k in ("bias", "gamma", "beta", "bias2"))
    T_out = c1g.out_len(c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K, stride=wl.stride,
                                      dilation=wl.dilation, pad_left=wl.pad_left,
                                      pad_right=wl.pad_right))
    odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    out = torch.full((wl.N, wl.C_out, T_out), float("nan") if poison else 0.0, device=DEV,
                     dtype=odt)
    if wl.norm is None and not wl.rowmin_bias:
        c1g.conv1d_forward(x, w, b, stride=wl.stride, dilation=wl.dilation,
                           pad_left=wl.pad_left, pad_right=wl.pad_right, out=out,
                           channels_last=wl.channels_last)
        res = (out, None, None)
    else:
        res = c1g.conv1d_gn_forward(x, w, b, stride=wl.stride, dilation=wl.dilation,
                                    pad_left=wl.pad_left, pad_right=wl.pad_right,
                                    norm=wl.norm, groups=wl.G, eps=wl.eps, gamma=ga, beta=be,
                                    rowmin_bias=b2, return_stats=True, out=out,
                                    persistent=wl.persistent, one_launch=wl.one_launch,
                                    cooperative=wl.cooperative,
                                    channels_last=wl.channels_last)
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


def library_route(wl: Workload):
    desc = c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K, stride=wl.stride,
                         dilation=wl.dilation, pad_left=wl.pad_left, pad_right=wl.pad_right,
                         dtype=c1g.C1G_BF16 if wl.dtype == "bf16" else c1g.C1G_F32,
                         out_dtype=c1g.C1G_BF16 if wl.out_dtype == "bf16" else c1g.C1G_F32,
                         x_layout=c1g.LAYOUT_NLC if wl.channels_last else c1g.LAYOUT_NCL)
    return c1g.route(desc, c1g.make_norm(wl.norm, wl.G, wl.eps, wl.rowmin_bias, wl.persistent,
                                         wl.one_launch, wl.cooperative))


def bf16_out_bound(wl: Workload, inp: dict, ref: dict):
    """Per-element bound on |out - oracle| for a bf16 output, derived from
    the arithmetic: the fp32-output tolerance tol, plus one rounding of the
    final value (BF16_U * (|ref| + tol)); on the split route y is stored
    rounded to bf16 before the normalisation reads it, which adds
    BF16_U * |y| * rstd * |gamma| (for the row-min, the largest such term over
    the channels of the position)."""
    tol = tol_for(wl)
    out = ref["out"]
    bound = tol + BF16_U * (np.abs(out) + tol)
    if library_route(wl) != "split":
        return bound
    y = np.abs(ref["y"])
    N, C, L = y.shape
    gam = np.ones(C) if inp["gamma"] is None else np.abs(to_f64_numpy(inp["gamma"]))
    if wl.norm == "group":
        rs = np.repeat(ref["rstd"], C // wl.G, axis=1)[:, :, None]       # [N, C, 1]
        scale = rs * gam[None, :, None]
    elif wl.norm == "layer_channels":
        scale = ref["rstd"][:, None, :] * gam[None, :, None]               # [N, C, L]
    else:
        scale = np.ones((1, C, 1))
    yterm = BF16_U * y * scale * (1 + 1e-3)
    if wl.rowmin_bias:
        yterm = np.broadcast_to(yterm.max(axis=1, keepdims=True), out.shape)
    return bound + yterm


def check_bf16_out(wl: Workload, got, inp: dict, ref: dict):
    """Element-wise |got - ref| <= bf16_out_bound; returns the worst ratio."""
    g = got.detach().to("cpu").to(torch.float64).numpy()
    assert g.shape == ref["out"].shape, (g.shape, ref["out"].shape)
    assert np.isfinite(g).all(), "non-finite output (unwritten element?)"
    ratio = np.abs(g - ref["out"]) / bf16_out_bound(wl, inp, ref)
    worst = float(ratio.max())
    assert worst <= 1.0, "%s: error %.3g x its bound at %s" % (
        wl.name, worst, np.unravel_index(int(ratio.argmax()), ratio.shape))
    return worst


def check_parity(wl: Workload, seed=0):
    announce(wl.name, wl, "seed", seed)
    inp = make_inputs(wl, seed)
    got, mean, rstd = run_library(wl, inp, return_stats=True)
    ref = run_oracle(wl, inp)
    if wl.out_dtype == "bf16":
        assert got.dtype == torch.bfloat16
        err = check_bf16_out(wl, got, inp, ref)
    else:
        err = max_abs_err(got, ref["out"])
        assert err <= tol_for(wl), "%s: max abs err %.3g > %.3g" % (wl.name, err, tol_for(wl))
    if mean is not None and ref["mean"] is not None:
        em = max_abs_err(mean, ref["mean"])
        er = float(np.max(np.abs(rstd.cpu().double().numpy() - ref["rstd"]) / ref["rstd"]))
        assert em <= 1e-4 * max(1.0, float(np.abs(ref["mean"]).max())), em
        assert er <= 1e-4, er
    return err
