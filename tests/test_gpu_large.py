"""Problems past 2^31 elements, up to the 2^32 limit of the boundary: every
offset the kernels form must hold such indices.  The outputs are checked
against the oracle on slices it can compute (whole GroupNorm groups of the
first and last sample: a group's statistics need only its own channels), and
the normalisation pass at the very limit (2^32 - 1 elements, an odd row
length so every element takes the scalar path) against float64 on the first
and last elements."""
import numpy as np
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
import oracle
from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs, to_f64_numpy
from tests.gpu_util import DEV, TOL_BF16, TOL_F32, announce, max_abs_err, to_dev

pytestmark = pytest.mark.gpu

LARGE = [
    # fp32, split route (conv with partial statistics, merge, apply in place)
    (Workload("large_split_fp32_gn", N=35, C_in=16, C_out=1024, T=60000, K=3, pad_left=1,
              pad_right=1, G=64), "split", TOL_F32),
    # bf16, persistent route, 256 tiles per sample
    (Workload("large_persistent_bf16_gn", N=130, C_in=64, C_out=1024, T=16384, K=3,
              pad_left=1, pad_right=1, G=32, dtype="bf16"), "fused_persistent", TOL_BF16),
    # fp32, single-pass route, 134400 workgroups
    (Workload("large_fused_fp32_gn", N=2100, C_in=16, C_out=1024, T=1024, K=3, pad_left=1,
              pad_right=1, G=64), "fused_single_pass", TOL_F32),
    # bf16 Linear + GroupNorm + row-min + bias (whole rows are checked)
    (Workload("large_gemm_rowmin", N=65535, C_in=64, C_out=40960, T=1, K=1, G=2560,
              rowmin_bias=True, dtype="bf16"), "gemm_rows", TOL_BF16),
]


@pytest.mark.parametrize("wl,route,tol", LARGE, ids=[c[0].name for c in LARGE])
def test_outputs_past_2_31(wl, route, tol):
    T_out = c1g.out_len(c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K,
                                      pad_left=wl.pad_left, pad_right=wl.pad_right))
    assert wl.N * wl.C_out * T_out > 2 ** 31
    announce("past 2^31 outputs", wl.name)
    inp = make_inputs(wl, 3)
    x, w = to_dev(inp["x"]), to_dev(inp["w"])
    b, ga, be, b2 = (to_dev(inp[k]) for k in ("bias", "gamma", "beta", "bias2"))
    op = c1g.PreparedConv1dGN(x, w, b, pad_left=wl.pad_left, pad_right=wl.pad_right,
                              norm="group", groups=wl.G, eps=wl.eps, gamma=ga, beta=be,
                              rowmin_bias=b2)
    assert op.route == route
    op.out.fill_(float("nan"))
    out = op()
    torch.cuda.synchronize()
    cpg = wl.C_out // wl.G
    f = to_f64_numpy
    for n, g in ((0, 0), (wl.N - 1, wl.G - 1)):
        # a whole group of sample n, or a whole row for the row-min
        c0, c1 = (0, wl.C_out) if wl.rowmin_bias else (g * cpg, (g + 1) * cpg)
        ref = oracle.forward(f(inp["x"][n:n + 1]), f(inp["w"][c0:c1]), f(inp["bias"][c0:c1]),
                             pad_left=wl.pad_left, pad_right=wl.pad_right, norm="group",
                             G=(c1 - c0) // cpg, eps=wl.eps, gamma=f(inp["gamma"][c0:c1]),
                             beta=f(inp["beta"][c0:c1]),
                             bias2=f(inp["bias2"][c0:c1]) if wl.rowmin_bias else None)
        err = max_abs_err(out[n:n + 1, c0:c1], ref["out"])
        assert err <= tol, (n, g, err)
    del op, out
    torch.cuda.empty_cache()


def test_gn_apply_at_the_index_limit():
    """y [1, 65535, 65537]: N*C*L = 2^32 - 1, the largest size gn_stats and
    gn_apply accept; L is odd, so gn_apply takes its scalar path, whose
    grid-strided counter must not wrap past 2^32.  The statistics of the first
    and last groups against float64; the first and last values after an
    in-place apply against float64."""
    N, C, L, G = 1, 65535, 65537, 5
    assert N * C * L == 2 ** 32 - 1
    announce("gn_stats / gn_apply at 2^32 - 1 elements")
    gen = torch.Generator(device=DEV).manual_seed(5)
    y = torch.randn((N, C, L), generator=gen, device=DEV)
    cpg = C // G
    ref = {}
    for g in (0, G - 1):
        v = y[0, g * cpg:(g + 1) * cpg].double()
        mu = v.mean()
        ref[g] = (float(mu), float(1.0 / torch.sqrt(((v - mu) ** 2).mean() + 1e-5)))
        del v
    k = 3 * L + 7  # the first and last values, across several rows
    head = y.view(-1)[:k].double().cpu().numpy()
    tail = y.view(-1)[-k:].double().cpu().numpy()
    gamma = torch.rand((C,), generator=gen, device=DEV) + 0.5
    beta = torch.randn((C,), generator=gen, device=DEV) * 0.1
    mean, rstd = c1g.gn_stats(y, G)
    c1g.gn_apply(y, mean, rstd, gamma, beta, groups=G, out=y)
    torch.cuda.synchronize()
    m, r = mean.double().cpu().numpy()[0], rstd.double().cpu().numpy()[0]
    for g, (mu, rs) in ref.items():
        assert abs(m[g] - mu) <= 1e-4 and abs(r[g] / rs - 1) <= 1e-4, (g, m[g], mu, r[g], rs)
    ga, be = gamma.double().cpu().numpy(), beta.double().cpu().numpy()
    for vals, start, got in ((head, 0, y.view(-1)[:k]), (tail, N * C * L - k, y.view(-1)[-k:])):
        e = start + np.arange(k)
        c = (e // L) % C
        g = c // cpg
        want = (vals - m[g]) * r[g] * ga[c] + be[c]
        err = float(np.abs(got.double().cpu().numpy() - want).max())
        assert err <= 1e-5, err
    del y
    torch.cuda.empty_cache()
