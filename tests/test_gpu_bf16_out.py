"""GPU parity of bf16 outputs (fp32 or bf16 inputs) against the fp64 oracle,
element by element, within a bound derived from the arithmetic: the fp32
output's tolerance plus bf16 rounding (one rounding of the final value; on the
split route also the rounding of the stored y that the normalisation reads)."""
import numpy as np
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
import oracle
from conv1d_implicit_gemm_amd.workloads import WORKLOADS, Workload, make_inputs
from tests.gpu_util import (BF16_U, TOL_F32, announce, check_bf16_out, check_parity,
                            library_route, run_library, run_oracle, to_dev)

pytestmark = pytest.mark.gpu

W = Workload
BO = dict(out_dtype="bf16")
CASES = [
    # bf16 inputs, split route: T_out % 8 == 4 (last unit of the vector apply),
    # then T_out % 4 != 0 (element-wise apply)
    (W("bf16o_conv_gn_k5d2", N=2, C_in=72, C_out=160, T=1300, K=5, dilation=2, pad_left=2,
       pad_right=2, G=8, dtype="bf16", persistent=False, **BO), "split"),
    (W("bf16o_conv_gn_k5d2_persistent", N=2, C_in=72, C_out=160, T=1300, K=5, dilation=2,
       pad_left=2, pad_right=2, G=8, dtype="bf16", **BO), "fused_persistent"),
    (W("bf16o_conv_gn_odd_T", N=2, C_in=40, C_out=64, T=203, K=3, pad_left=1, pad_right=1,
       G=4, dtype="bf16", **BO), "fused_persistent"),
    (W("bf16o_conv_gn_odd_T_split", N=2, C_in=40, C_out=64, T=203, K=3, pad_left=1,
       pad_right=1, G=4, dtype="bf16", persistent=False, **BO), "split"),
    (W("bf16o_conv_ln", N=1, C_in=40, C_out=272, T=1300, K=5, dilation=2, pad_left=2,
       pad_right=2, norm="layer_channels", dtype="bf16", **BO), "fused_persistent"),
    (W("bf16o_conv_ln_split", N=1, C_in=40, C_out=272, T=1300, K=5, dilation=2, pad_left=2,
       pad_right=2, norm="layer_channels", dtype="bf16", persistent=False, **BO), "split"),
    (W("bf16o_conv_gn_rowmin", N=2, C_in=32, C_out=64, T=96, K=3, pad_left=1, pad_right=1,
       G=4, rowmin_bias=True, dtype="bf16", **BO), "split"),
    (W("bf16o_conv_ln_rowmin", N=2, C_in=32, C_out=48, T=70, K=3, pad_left=1, pad_right=1,
       norm="layer_channels", rowmin_bias=True, dtype="bf16", **BO), "split"),
    (W("bf16o_conv_only", N=3, C_in=48, C_out=130, T=256, K=2, norm=None, dtype="bf16", **BO),
     "conv_only"),
    (W("bf16o_conv_gn_k8", N=2, C_in=48, C_out=144, T=300, K=8, pad_left=3, pad_right=4, G=9,
       dtype="bf16", **BO), "fused_persistent"),
    # fp32 inputs
    (W("f32in_bf16o_fused_gn", N=2, C_in=64, C_out=128, T=512, K=3, pad_left=1, pad_right=1,
       G=16, **BO), "fused_single_pass"),
    (W("f32in_bf16o_fused_gn_ragged", N=3, C_in=20, C_out=40, T=301, K=3, pad_left=1,
       pad_right=1, G=5, **BO), "fused_single_pass"),
    (W("f32in_bf16o_split_gn", N=2, C_in=24, C_out=64, T=2000, K=3, pad_left=1, pad_right=1,
       G=2, **BO), "split"),
    (W("f32in_bf16o_causal", N=2, C_in=32, C_out=48, T=515, K=4, pad_left=3, norm=None,
       bias=False, affine=False, w_bound=1.0 / 32.0, **BO), "conv_only"),
    # the Linear-layer GEMM route, every epilogue
    (W("gemm_bf16o_gn_rowmin_fused", N=70, C_in=256, C_out=512, T=1, K=1, G=32, bias=False,
       rowmin_bias=True, dtype="bf16", **BO), "gemm_rows"),
    (W("gemm_bf16o_gn", N=33, C_in=96, C_out=128, T=1, K=1, G=8, dtype="bf16", **BO),
     "gemm_rows"),
    (W("gemm_bf16o_ln", N=33, C_in=96, C_out=200, T=1, K=1, norm="layer_channels",
       dtype="bf16", **BO), "gemm_rows"),
    (W("gemm_bf16o_only", N=50, C_in=64, C_out=300, T=1, K=1, norm=None, dtype="bf16", **BO),
     "gemm_rows"),
    (W("gemm_bf16o_gn_rowmin_unfused", N=20, C_in=64, C_out=96, T=1, K=1, G=3,
       rowmin_bias=True, dtype="bf16", **BO), "gemm_rows"),
    (W("gemm_bf16o_gn_rowmin_one_launch", N=200, C_in=128, C_out=528, T=1, K=1, G=33,
       rowmin_bias=True, dtype="bf16", one_launch=True, **BO), "gemm_rows"),
]


@pytest.mark.parametrize("wl,route", CASES, ids=lambda c: getattr(c, "name", c))
def test_bf16_out_parity(wl, route):
    assert library_route(wl) == route
    check_parity(wl)


def test_bf16_out_matches_rounded_fp32_out():
    """Where only the final value is rounded (fused, persistent and GEMM
    routes), the bf16 output is the fp32 output rounded to nearest even, bit
    for bit (same kernels, same fp32 arithmetic)."""
    by_name = {wl.name: wl for wl, _ in CASES}
    for name in ("f32in_bf16o_fused_gn", "gemm_bf16o_gn_rowmin_fused", "gemm_bf16o_only",
                 "gemm_bf16o_gn_rowmin_one_launch", "bf16o_conv_gn_odd_T", "bf16o_conv_ln"):
        wl = by_name[name]
        announce("bf16 out == rne(fp32 out)", wl.name)
        inp = make_inputs(wl, 1)
        got = run_library(wl, inp)
        f32 = run_library(wl.replace(out_dtype="f32"), inp)
        assert torch.equal(got.view(torch.int16), f32.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("name", ["conv1d_gn_bf16_n64_c512x1024_t4096_k5d2",
                                  "conv1d_lnc_bf16_n64_c512x1024_t4096_k5d2"])
def test_bf16_out_full_size_sampled(name):
    """The bf16 dilated-conv workload at full size with a bf16 output; the
    oracle checks two whole samples (statistics are per sample)."""
    wl = WORKLOADS[name].replace(out_dtype="bf16")
    announce(wl.name, "bf16 out")
    inp = make_inputs(wl, 0)
    got = run_library(wl, inp)
    for n in (0, wl.N - 1):
        ref = run_oracle(wl, inp, n_slice=slice(n, n + 1))
        sub = dict(inp)
        check_bf16_out(wl.replace(N=1), got[n:n + 1], sub, ref)


def test_gn_apply_bf16_standalone():
    """gn_apply_bf16 (and in place) vs the oracle's GroupNorm of the same bf16
    values, using gn_stats of the widened values; bound: fp32 arithmetic plus
    one rounding of the result."""
    announce("gn_apply_bf16")
    g = torch.Generator().manual_seed(7)
    for (N, C, L, G) in [(2, 32, 1000, 8), (3, 24, 77, 8), (1, 16, 4092, 4), (2, 16, 4093, 4),
                         (4, 12, 1, 3)]:
        y = (torch.randn(N, C, L, generator=g) * 2 + 0.5).to(torch.bfloat16)
        gam = torch.rand(C, generator=g) + 0.5
        bet = torch.randn(C, generator=g) * 0.1
        z_ref, _, _ = oracle.group_norm(y.double().numpy(), G, 1e-5, gam.double().numpy(),
                                        bet.double().numpy())
        yd = to_dev(y)
        mean, rstd = c1g.gn_stats(yd.float(), G, 1e-5)
        out = c1g.gn_apply(yd, mean, rstd, to_dev(gam), to_dev(bet), groups=G)
        torch.cuda.synchronize()
        assert out.dtype == torch.bfloat16
        err = np.abs(out.cpu().double().numpy() - z_ref)
        bound = TOL_F32 + BF16_U * (np.abs(z_ref) + TOL_F32)
        assert (err <= bound).all(), (N, C, L, G, float((err / bound).max()))
        c1g.gn_apply(yd, mean, rstd, to_dev(gam), to_dev(bet), groups=G, out=yd)  # in place
        torch.cuda.synchronize()
        assert torch.equal(yd.view(torch.int16), out.view(torch.int16))


def test_bf16_out_determinism():
    wl = CASES[0][0]
    announce("bf16 out determinism")
    inp = make_inputs(wl, 4)
    assert torch.equal(run_library(wl, inp).view(torch.int16),
                       run_library(wl, inp).view(torch.int16))
