"""A NaN or an infinity in the input stays where the definition puts it.

One element of x (sample n0, input channel c0, position t0) is set to NaN
(or +inf: the same elements become non-finite, and the GPU and the oracle
agree on which of them are NaN, +inf or -inf).
The convolution carries it into every output channel at the output
positions whose window holds t0 (t·s + j·d − p_l = t0 for some tap j); a
GroupNorm group's statistics cover all positions of its channels, so under
GroupNorm the whole sample becomes NaN; a LayerNorm over channels keeps it
at those positions; the row-min reduces like PyTorch's min over the channel
dimension (the model of "Kimi-K2.6 l2_p75"), which returns NaN for a row
holding one.  Each case checks, on every route, that the output is
non-finite exactly there, that every other value has the bits of the clean
run (no statistics, staging or rounds shared across samples or positions
leak it), and that the oracle marks the same elements NaN, +inf or -inf and
agrees on the poisoned sample's finite values."""
import numpy as np
import pytest
import torch

from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import (TOL_BF16, TOL_F32, announce, library_route, run_library,
                            run_oracle)

pytestmark = pytest.mark.gpu

BF = dict(dtype="bf16")
# (workload, route, n0, c0, t0)
CASES = [
    (Workload("nan_fused_f32_gn", N=4, C_in=32, C_out=64, T=300, K=3, pad_left=1, pad_right=1,
              G=8), "fused_single_pass", 1, 5, 150),
    (Workload("nan_split_f32_gn", N=3, C_in=24, C_out=48, T=1500, K=3, pad_left=1,
              pad_right=1, G=6), "split", 2, 0, 0),
    (Workload("nan_split_f32_ln", N=3, C_in=24, C_out=48, T=1500, K=5, dilation=2, pad_left=4,
              pad_right=4, norm="layer_channels"), "split", 1, 23, 777),
    (Workload("nan_conv_only_f32", N=3, C_in=24, C_out=48, T=700, K=4, pad_left=3, norm=None),
     "conv_only", 0, 7, 699),
    (Workload("nan_split_f32_rowmin_nonorm", N=3, C_in=24, C_out=48, T=200, K=4, pad_left=3,
              norm=None, rowmin_bias=True), "split", 1, 3, 100),
    (Workload("nan_split_f32_gn_rowmin", N=3, C_in=24, C_out=48, T=200, K=4, pad_left=3, G=6,
              rowmin_bias=True), "split", 2, 11, 3),
    (Workload("nan_linear_f32_gn_rowmin", N=40, C_in=64, C_out=96, T=1, K=1, G=6,
              rowmin_bias=True), "split", 17, 63, 0),
    (Workload("nan_persistent_bf16_gn", N=14, C_in=64, C_out=512, T=2200, K=3, pad_left=1,
              pad_right=1, G=32, **BF), "fused_persistent", 0, 9, 1000),
    (Workload("nan_persistent_bf16_ln", N=14, C_in=64, C_out=512, T=2200, K=3, pad_left=1,
              pad_right=1, norm="layer_channels", **BF), "fused_persistent", 0, 63, 511),
    (Workload("nan_split_bf16_gn", N=3, C_in=72, C_out=160, T=1300, K=5, dilation=2,
              pad_left=2, pad_right=2, G=8, persistent=False, **BF), "split", 1, 40, 640),
    (Workload("nan_gemm_rowmin", N=300, C_in=256, C_out=512, T=1, K=1, G=32, rowmin_bias=True,
              **BF), "gemm_rows", 131, 200, 0),
    (Workload("nan_gemm_rowmin_one_launch", N=300, C_in=256, C_out=512, T=1, K=1, G=32,
              rowmin_bias=True, one_launch=True, **BF), "gemm_rows", 299, 0, 0),
    (Workload("nan_gemm_gn32_rowmin", N=300, C_in=256, C_out=512, T=1, K=1, G=16,
              rowmin_bias=True, **BF), "gemm_rows", 5, 255, 0),
]


def expected_nan(wl, T_out, n0, t0):
    """[N, C_out, T_out] mask of the outputs the definition makes NaN."""
    hit = np.zeros(T_out, dtype=bool)
    for t in range(T_out):
        for j in range(wl.K):
            if t * wl.stride + j * wl.dilation - wl.pad_left == t0:
                hit[t] = True
    mask = np.zeros((wl.N, wl.C_out, T_out), dtype=bool)
    if wl.norm == "group":  # every group's statistics see the NaN positions
        mask[n0] = hit.any()
    else:  # no norm, or LayerNorm over channels: those positions, every channel
        mask[n0, :, hit] = True
    return mask


@pytest.mark.parametrize("poison", [float("nan"), float("inf")], ids=["nan", "inf"])
@pytest.mark.parametrize("wl,route,n0,c0,t0", CASES, ids=[c[0].name for c in CASES])
def test_nan_stays_where_defined(wl, route, n0, c0, t0, poison):
    announce("non-finite propagation", wl.name, poison)
    assert library_route(wl) == route
    inp = make_inputs(wl, 21)
    clean = run_library(wl, inp).cpu()
    bad = dict(inp)
    bad["x"] = inp["x"].clone()
    bad["x"][n0, c0, t0] = poison
    got = run_library(wl, bad).cpu()
    mask = expected_nan(wl, got.shape[2], n0, t0)
    assert mask.any()
    assert torch.isfinite(clean).all()
    assert np.array_equal(~torch.isfinite(got).numpy(), mask)
    m = torch.from_numpy(mask)
    assert torch.equal(got[~m], clean[~m])
    # the oracle on the poisoned sample: the same NaN elements, the same
    # finite values within tolerance
    ref = run_oracle(wl, bad, n_slice=slice(n0, n0 + 1))["out"]
    assert np.array_equal(~np.isfinite(ref), mask[n0:n0 + 1])
    g = got[n0:n0 + 1].double().numpy()
    for kind in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(kind(g), kind(ref)), kind.__name__
    ok = ~mask[n0:n0 + 1]
    if ok.any():
        err = float(np.abs(got[n0:n0 + 1].double().numpy()[ok] - ref[ok]).max())
        assert err <= (TOL_BF16 if wl.dtype == "bf16" else TOL_F32), err
