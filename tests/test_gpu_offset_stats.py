"""Statistics of values whose mean is far larger than their spread.

Every channel's conv bias is shifted by a constant (64 on the fp32 routes,
1024 on the bf16 ones), so each GroupNorm group and each LayerNorm position
has a mean of about that size and a standard deviation of about 1.  The
normalisation must still match the oracle to the usual tolerance: the
kernels take exact two-pass statistics (the mean, then squared deviations
from it) and merge them with Chan's update, whereas a single pass over sums
of squares (E[y^2] - E[y]^2) in fp32 misses the variance of 8192 such values
by ~4e-4 (relative) at a shift of 64 and by 2-25% at 1024 (fp32 sums of 16
values, then a tree), beyond the 1e-4 relative bound on rstd.  The
standalone gn_stats / gn_apply on y = 1000 + N(0, 1) are checked against
float64 the same way."""
import numpy as np
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import (DEV, TOL_BF16, TOL_F32, announce, library_route, max_abs_err,
                            run_library, run_oracle)

pytestmark = pytest.mark.gpu

BF = dict(dtype="bf16")
# (workload, route, bias shift)
CASES = [
    (Workload("shift_fused_f32_gn", N=4, C_in=32, C_out=64, T=1024, K=3, pad_left=1,
              pad_right=1, G=8), "fused_single_pass", 64.0),
    (Workload("shift_split_f32_gn", N=3, C_in=24, C_out=48, T=1500, K=3, pad_left=1,
              pad_right=1, G=6), "split", 64.0),
    (Workload("shift_split_f32_ln", N=3, C_in=24, C_out=48, T=1500, K=5, dilation=2,
              pad_left=4, pad_right=4, norm="layer_channels"), "split", 64.0),
    (Workload("shift_linear_f32_gn_rowmin", N=40, C_in=64, C_out=96, T=1, K=1, G=6,
              rowmin_bias=True), "split", 64.0),
    (Workload("shift_persistent_bf16_gn", N=5, C_in=64, C_out=512, T=2200, K=3, pad_left=1,
              pad_right=1, G=32, **BF), "fused_persistent", 1024.0),
    (Workload("shift_persistent_bf16_ln", N=5, C_in=64, C_out=512, T=2200, K=3, pad_left=1,
              pad_right=1, norm="layer_channels", **BF), "fused_persistent", 1024.0),
    (Workload("shift_split_bf16_gn", N=3, C_in=72, C_out=160, T=1300, K=5, dilation=2,
              pad_left=2, pad_right=2, G=8, persistent=False, **BF), "split", 1024.0),
    (Workload("shift_gemm_gn16_rowmin", N=300, C_in=256, C_out=512, T=1, K=1, G=32,
              rowmin_bias=True, **BF), "gemm_rows", 1024.0),
    (Workload("shift_gemm_gn32", N=300, C_in=256, C_out=512, T=1, K=1, G=16, **BF),
     "gemm_rows", 1024.0),
]


@pytest.mark.parametrize("wl,route,shift", CASES, ids=[c[0].name for c in CASES])
def test_shifted_statistics(wl, route, shift):
    announce("shifted statistics", wl.name, shift)
    assert library_route(wl) == route
    inp = make_inputs(wl, 31)
    inp = dict(inp, bias=inp["bias"] + shift)
    got, mean, rstd = run_library(wl, inp, return_stats=True)
    ref = run_oracle(wl, inp)
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_F32
    err = max_abs_err(got, ref["out"])
    assert err <= tol, err
    if mean is not None and ref["mean"] is not None:
        assert float(np.abs(ref["mean"]).min()) > shift / 2  # the shift took hold
        assert max_abs_err(mean, ref["mean"]) <= 1e-4 * shift
        r = rstd.cpu().double().numpy()
        assert float(np.max(np.abs(r / ref["rstd"] - 1))) <= 1e-4


def test_shifted_gn_stats_and_apply():
    """gn_stats and gn_apply on y = 1000 + N(0, 1), [4, 64, 4096], G 8:
    statistics against float64 of the same fp32 values, and the applied
    values against float64."""
    gen = torch.Generator(device=DEV).manual_seed(4)
    y = torch.randn((4, 64, 4096), generator=gen, device=DEV) + 1000.0
    announce("shifted gn_stats / gn_apply")
    G = 8
    mean, rstd = c1g.gn_stats(y, G)
    out = c1g.gn_apply(y, mean, rstd, groups=G)
    torch.cuda.synchronize()
    yd = y.double().cpu().view(4, G, -1)
    mu = yd.mean(dim=2)
    rs = 1.0 / torch.sqrt(((yd - mu[:, :, None]) ** 2).mean(dim=2) + 1e-5)
    assert float((mean.double().cpu() - mu).abs().max()) <= 1e-3  # 16 ulps at 1000
    assert float((rstd.double().cpu() / rs - 1).abs().max()) <= 1e-4
    want = ((yd - mu[:, :, None]) * rs[:, :, None]).view(4, 64, 4096)
    assert float((out.double().cpu() - want).abs().max()) <= 2e-3
