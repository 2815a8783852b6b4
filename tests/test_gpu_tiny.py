"""The smallest problems each route accepts, against the oracle: one input or
output channel, one position, one tap, windows wider than the input, stride
that leaves a single output position, and the degenerate statistics they
bring (a GroupNorm group or a LayerNorm position of one value has variance
0, so its output is beta: the pages' definition with the population
variance and eps inside the root)."""
import numpy as np
import pytest

from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import announce, check_parity, library_route, run_library

pytestmark = pytest.mark.gpu

BF = dict(dtype="bf16")
CASES = [
    # fp32 single pass: one channel in and out, one position
    (Workload("tiny_fused_1x1x1", N=1, C_in=1, C_out=1, T=1, K=1, G=1), "fused_single_pass"),
    # a window wider than the input (K 5 over T 2, padded)
    (Workload("tiny_fused_k_gt_t", N=2, C_in=3, C_out=4, T=2, K=5, pad_left=2, pad_right=2,
              G=4), "fused_single_pass"),
    # stride leaves one output position
    (Workload("tiny_split_stride_tout1", N=2, C_in=5, C_out=3, T=5, K=5, stride=3, G=3),
     "split"),
    # fp32 LayerNorm over a single channel
    (Workload("tiny_split_ln_c1", N=2, C_in=2, C_out=1, T=40, K=3, pad_left=1, pad_right=1,
              norm="layer_channels"), "split"),
    (Workload("tiny_split_c1_long", N=1, C_in=1, C_out=1, T=2000, K=3, pad_left=2, G=1),
     "split"),
    (Workload("tiny_conv_only_f32", N=1, C_in=1, C_out=1, T=3, K=4, pad_left=3, norm=None),
     "conv_only"),
    (Workload("tiny_rowmin_c1", N=2, C_in=1, C_out=1, T=9, K=2, pad_left=1, G=1,
              rowmin_bias=True), "split"),
    # bf16
    (Workload("tiny_bf16_persistent_ln_c1", N=1, C_in=1, C_out=1, T=7, K=3, pad_left=1,
              pad_right=1, norm="layer_channels", **BF), "fused_persistent"),
    (Workload("tiny_bf16_persistent_gn_g1", N=1, C_in=1, C_out=2, T=1, K=1, G=1, **BF),
     "fused_persistent"),
    (Workload("tiny_bf16_conv_only", N=1, C_in=1, C_out=1, T=1, K=1, norm=None, **BF),
     "conv_only"),
    (Workload("tiny_bf16_split_k8", N=1, C_in=2, C_out=3, T=3, K=8, pad_left=4, pad_right=3,
              G=3, persistent=False, **BF), "split"),
    # the Linear route: one row, one output channel
    (Workload("tiny_gemm_1x8x1", N=1, C_in=8, C_out=1, T=1, K=1, G=1, **BF), "gemm_rows"),
    (Workload("tiny_gemm_rowmin", N=1, C_in=8, C_out=16, T=1, K=1, G=1, rowmin_bias=True,
              **BF), "gemm_rows"),
]


@pytest.mark.parametrize("wl,route", CASES, ids=[c[0].name for c in CASES])
def test_tiny(wl, route):
    assert library_route(wl) == route
    check_parity(wl)


@pytest.mark.parametrize("wl,route", [c for c in CASES if c[0].name in
                                      ("tiny_fused_1x1x1", "tiny_split_ln_c1",
                                       "tiny_bf16_persistent_ln_c1", "tiny_gemm_1x8x1")],
                         ids=lambda c: getattr(c, "name", c))
def test_single_value_statistics_give_beta(wl, route):
    """A group or position of one value: (y - mean) is exactly 0, so the
    output is beta exactly."""
    announce("single-value statistics", wl.name)
    inp = make_inputs(wl, 5)
    got = run_library(wl, inp).cpu().double().numpy()
    beta = inp["beta"].double().numpy()
    assert np.array_equal(got, np.broadcast_to(beta[None, :, None], got.shape))
