"""Channels-last input (x handed over as [N, T, C_in]) on every route: parity
against the oracle, which reads the same values as [N, C_in, T], and results
bit-identical to the channels-first call (the bf16 routes build the same
input image, the fp32 routes run the same kernels on the transposed copy)."""
import pytest
import torch

from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import announce, check_parity, library_route, run_library

pytestmark = pytest.mark.gpu

W = Workload
NLC = dict(channels_last=True)
BF = dict(dtype="bf16", **NLC)
# (workload, route); channel counts that are not multiples of the 64-wide
# transpose tile or of the 8-channel image pieces exercise the ragged paths
CASES = [
    (W("nlc_f32_fused_gn", N=2, C_in=16, C_out=32, T=256, K=3, pad_left=1, pad_right=1, G=8,
       **NLC), "fused_single_pass"),
    (W("nlc_f32_split_gn", N=2, C_in=24, C_out=64, T=2000, K=3, pad_left=1, pad_right=1, G=2,
       **NLC), "split"),
    (W("nlc_f32_ln_ragged_C", N=2, C_in=70, C_out=96, T=300, K=5, dilation=2, pad_left=4,
       pad_right=4, norm="layer_channels", **NLC), "split"),
    (W("nlc_f32_causal_conv_only", N=2, C_in=40, C_out=48, T=515, K=4, pad_left=3, norm=None,
       bias=False, **NLC), "conv_only"),
    (W("nlc_bf16_persist_gn", N=3, C_in=72, C_out=256, T=1300, K=5, dilation=2, pad_left=4,
       pad_right=4, G=16, **BF), "fused_persistent"),
    (W("nlc_bf16_persist_ln_bf16_out", N=2, C_in=64, C_out=128, T=700, K=3, pad_left=1,
       pad_right=1, norm="layer_channels", out_dtype="bf16", **BF), "fused_persistent"),
    (W("nlc_bf16_split_rowmin", N=2, C_in=32, C_out=64, T=96, K=3, pad_left=1, pad_right=1, G=4,
       rowmin_bias=True, **BF), "split"),
    (W("nlc_bf16_conv_only_C37", N=2, C_in=37, C_out=64, T=300, K=3, pad_left=1, pad_right=1,
       norm=None, **BF), "conv_only"),
    (W("nlc_bf16_stride3_gn", N=2, C_in=33, C_out=48, T=401, K=3, stride=3, pad_left=1,
       pad_right=1, G=6, **BF), "fused_persistent"),
    (W("nlc_bf16_k8_gn", N=2, C_in=48, C_out=144, T=300, K=8, pad_left=3, pad_right=4, G=9,
       **BF), "fused_persistent"),
    (W("nlc_bf16_k8_gn_split", N=2, C_in=48, C_out=144, T=300, K=8, pad_left=3, pad_right=4,
       G=9, persistent=False, **BF), "split"),
    (W("nlc_bf16_linear_gn_rowmin", N=70, C_in=256, C_out=512, T=1, K=1, G=32,
       rowmin_bias=True, **BF), "gemm_rows"),
]


@pytest.mark.parametrize("wl,route", CASES, ids=lambda c: getattr(c, "name", c))
def test_channels_last_parity(wl, route):
    assert library_route(wl) == route
    check_parity(wl)


@pytest.mark.parametrize("wl,route", CASES, ids=lambda c: getattr(c, "name", c))
def test_channels_last_matches_channels_first(wl, route):
    announce("channels-last == channels-first", wl.name)
    inp = make_inputs(wl, 6)
    a = run_library(wl, inp, return_stats=True)
    b = run_library(wl.replace(channels_last=False), inp, return_stats=True)
    for u, v in zip(a, b):
        assert (u is None) == (v is None)
        if u is not None:
            assert torch.equal(u, v)
