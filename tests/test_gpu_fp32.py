"""GPU parity of the fp32 path against the fp64 oracle (element by element,
max-abs 1e-4 after normalisation), plus the properties the pages fix that can
be checked bit-exactly on the device: causality, the delta kernel and
run-to-run determinism."""
import numpy as np
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
import oracle
from conv1d_implicit_gemm_amd.workloads import WORKLOADS, Workload, make_inputs, to_f64_numpy
from tests.gpu_util import (DEV, TOL_F32, announce, check_parity, max_abs_err, run_library,
                            run_oracle, to_dev)

pytestmark = pytest.mark.gpu

W = Workload
# Shapes that span several tiles and end in ragged tails (tile: 128 positions x
# 128 channels, 8 input channels per K-chunk), every route, and the edge cases.
CONV_CASES = [
    W("conv_ragged_k3", N=2, C_in=19, C_out=150, T=300, K=3, pad_left=1, pad_right=1,
      norm=None),
    W("conv_causal_k4", N=2, C_in=24, C_out=40, T=515, K=4, pad_left=3, pad_right=0, norm=None,
      bias=False),
    W("conv_stride2_d3", N=3, C_in=9, C_out=130, T=701, K=5, stride=2, dilation=3, pad_left=4,
      pad_right=1, norm=None),
    W("conv_stride3", N=1, C_in=5, C_out=7, T=1000, K=2, stride=3, norm=None),
    W("conv_k1", N=2, C_in=33, C_out=17, T=129, K=1, norm=None),
    W("conv_k1_t1", N=37, C_in=40, C_out=65, T=1, K=1, norm=None),
    W("conv_odd_T", N=2, C_in=7, C_out=9, T=131, K=3, pad_left=1, pad_right=1, norm=None),
    W("conv_no_pad_short", N=1, C_in=3, C_out=5, T=6, K=4, norm=None),
    W("conv_k8", N=1, C_in=16, C_out=20, T=200, K=8, pad_left=7, norm=None),
]


@pytest.mark.parametrize("wl", CONV_CASES, ids=lambda w: w.name)
def test_conv_parity(wl):
    check_parity(wl)


GN_CASES = [
    WORKLOADS["conv1d_gn_f32_n2_c16x32_t256_k3"],
    WORKLOADS["conv1d_gn_f32_n16_c128x256_t1024_k3"],
    # fused route: ragged T_out, channel count not a multiple of 16, cpg 1/2/16
    W("fused_ragged", N=3, C_in=10, C_out=24, T=333, K=3, pad_left=1, pad_right=1, G=6),
    W("fused_cpg1", N=2, C_in=8, C_out=16, T=100, K=2, G=16),
    W("fused_cpg16", N=2, C_in=12, C_out=48, T=517, K=3, dilation=2, pad_left=2, pad_right=2,
      G=3),
    W("fused_no_affine_no_bias", N=1, C_in=4, C_out=8, T=64, K=3, G=2, bias=False,
      affine=False),
    W("fused_t1", N=4, C_in=40, C_out=32, T=1, K=1, G=4),
    # more of the fused route: a partial last 16-channel chunk, a single chunk,
    # 8 taps at dilation 2 (causal), dilation 3 with 13 chunks, many chunks,
    # and a halo of 18 positions
    W("fused_cin20_t512", N=2, C_in=20, C_out=32, T=512, K=3, pad_left=1, pad_right=1, G=8),
    W("fused_one_chunk_k5", N=2, C_in=5, C_out=16, T=64, K=5, pad_left=2, pad_right=2, G=4),
    W("fused_k8d2_causal", N=1, C_in=16, C_out=16, T=256, K=8, dilation=2, pad_left=14, G=2),
    W("fused_k5d3_cin100", N=2, C_in=100, C_out=32, T=1024, K=5, dilation=3, pad_left=6,
      pad_right=6, G=4),
    W("fused_cin256", N=2, C_in=256, C_out=32, T=1024, K=3, pad_left=1, pad_right=1, G=4),
    W("fused_k4d6_halo18", N=1, C_in=16, C_out=16, T=1024, K=4, dilation=6, pad_left=9,
      pad_right=9, G=2),
    # split route: C_out/G not a divisor of 16, or T_out beyond the on-chip slab
    W("split_cpg3", N=2, C_in=20, C_out=24, T=300, K=3, pad_left=1, pad_right=1, G=8),
    W("split_long", N=2, C_in=16, C_out=32, T=1500, K=3, pad_left=1, pad_right=1, G=8),
    W("split_stride2", N=2, C_in=9, C_out=40, T=500, K=4, stride=2, G=5),
    W("split_cpg24_ctile_straddle", N=2, C_in=17, C_out=240, T=130, K=3, pad_left=1,
      pad_right=1, G=10),
    # a single group over every channel
    W("split_g1", N=2, C_in=12, C_out=48, T=300, K=3, pad_left=1, pad_right=1, G=1),
]


@pytest.mark.parametrize("wl", GN_CASES, ids=lambda w: w.name)
def test_groupnorm_parity(wl):
    check_parity(wl)


LN_ROWMIN_CASES = [
    W("ln_channels", N=2, C_in=12, C_out=160, T=200, K=3, pad_left=1, pad_right=1,
      norm="layer_channels"),
    W("ln_channels_t1", N=5, C_in=12, C_out=40, T=1, K=1, norm="layer_channels"),
    W("gn_rowmin_t1", N=64, C_in=96, C_out=256, T=1, K=1, G=16, bias=False, rowmin_bias=True),
    W("gn_rowmin_t", N=2, C_in=8, C_out=48, T=70, K=3, pad_left=1, pad_right=1, G=4,
      rowmin_bias=True),
    W("ln_rowmin", N=2, C_in=8, C_out=48, T=70, K=3, pad_left=1, pad_right=1,
      norm="layer_channels", rowmin_bias=True),
    W("rowmin_only", N=3, C_in=8, C_out=20, T=33, K=3, norm=None, rowmin_bias=True),
]


@pytest.mark.parametrize("wl", LN_ROWMIN_CASES, ids=lambda w: w.name)
def test_ln_rowmin_parity(wl):
    check_parity(wl)


def test_causal_conv_full_size_sampled():
    """The causal workload at full size; the oracle checks two whole samples
    (the first and the last) element by element."""
    wl = WORKLOADS["causal_conv1d_f32_n32_c256x256_t8192_k4"]
    announce(wl.name)
    inp = make_inputs(wl, 0)
    got = run_library(wl, inp)
    for n in (0, wl.N - 1):
        ref = run_oracle(wl, inp, n_slice=slice(n, n + 1))
        err = max_abs_err(got[n:n + 1], ref["out"])
        assert err <= TOL_F32, (n, err)


def test_causality_bitwise():
    """Perturbing x after t0 leaves y[..., :t0+1] bit-identical on the device."""
    wl = W("causal", N=2, C_in=20, C_out=36, T=400, K=4, pad_left=3, pad_right=0, norm=None)
    announce("causality")
    inp = make_inputs(wl, 1)
    y0 = run_library(wl, inp)
    for t0 in (0, 127, 128, 250):
        inp2 = dict(inp)
        x2 = inp["x"].clone()
        x2[:, :, t0 + 1:] += torch.randn(x2[:, :, t0 + 1:].shape) * 5
        inp2["x"] = x2
        y1 = run_library(wl, inp2)
        assert torch.equal(y0[:, :, :t0 + 1], y1[:, :, :t0 + 1]), t0
        assert not torch.equal(y0[:, :, t0 + 1:], y1[:, :, t0 + 1:])


@pytest.mark.parametrize("K,s,d,pl,pr", [(4, 1, 1, 3, 0), (3, 2, 2, 1, 2), (5, 1, 3, 6, 6)])
def test_delta_kernel_bitwise(K, s, d, pl, pr):
    """w[c,ci,j] = [c==ci][j==j0]: y is x read at t*s + j0*d - pl, exactly."""
    announce("delta", K, s, d, pl, pr)
    C, T = 20, 300
    x = torch.randn(2, C, T)
    for j0 in range(K):
        w = torch.zeros(C, C, K)
        w[torch.arange(C), torch.arange(C), j0] = 1.0
        y = c1g.conv1d_forward(to_dev(x), to_dev(w), stride=s, dilation=d, pad_left=pl,
                               pad_right=pr).cpu()
        T_out = y.shape[2]
        u = torch.arange(T_out) * s + j0 * d - pl
        valid = (u >= 0) & (u < T)
        want = torch.zeros(2, C, T_out)
        want[:, :, valid] = x[:, :, u[valid]]
        assert torch.equal(y, want), j0


@pytest.mark.parametrize("name", ["conv1d_gn_f32_n16_c128x256_t1024_k3", "split_cpg3"])
def test_determinism(name):
    wl = WORKLOADS.get(name) or next(w for w in GN_CASES if w.name == name)
    announce("determinism", name)
    inp = make_inputs(wl, 3)
    a = run_library(wl, inp)
    b = run_library(wl, inp)
    assert torch.equal(a, b)


def test_gn_stats_and_apply_standalone():
    """gn_stats + gn_apply on an existing y (and in place) vs the oracle's GroupNorm."""
    announce("gn_stats/gn_apply")
    g = torch.Generator().manual_seed(5)
    # groups of up to 32768 values (one workgroup each), then groups cut into
    # several slices merged in a second stage: one group over a whole sample
    # (N * G = 1), a ragged last slice, and a length that is no multiple of 4
    # (the unvectorised loads)
    for (N, C, L, G) in [(2, 32, 1000, 8), (3, 24, 77, 8), (1, 16, 4093, 4), (4, 12, 1, 3),
                         (1, 64, 4096, 1), (2, 96, 2000, 2), (1, 35, 3001, 1),
                         (2, 1024, 4092, 32)]:
        y = torch.randn(N, C, L, generator=g) * 2 + 0.5
        gam = torch.rand(C, generator=g) + 0.5
        bet = torch.randn(C, generator=g) * 0.1
        z_ref, m_ref, r_ref = oracle.group_norm(y.double().numpy(), G, 1e-5,
                                                gam.double().numpy(), bet.double().numpy())
        yd = to_dev(y)
        mean, rstd = c1g.gn_stats(yd, G, 1e-5)
        assert max_abs_err(mean, m_ref) <= 1e-5
        assert float(np.max(np.abs(rstd.cpu().double().numpy() / r_ref - 1))) <= 1e-5
        out = c1g.gn_apply(yd, mean, rstd, to_dev(gam), to_dev(bet), groups=G)
        assert max_abs_err(out, z_ref) <= TOL_F32
        c1g.gn_apply(yd, mean, rstd, to_dev(gam), to_dev(bet), groups=G, out=yd)  # in place
        assert torch.equal(yd, out)


def test_gn_stats_two_stage_deterministic_and_unaligned():
    """gn_stats on groups of several slices: bit-identical from run to run, and
    the same values (to rounding) when y starts 4 bytes off a 16-byte
    boundary, which takes the unvectorised loads."""
    announce("gn_stats two-stage determinism / unaligned y")
    g = torch.Generator().manual_seed(11)
    N, C, L, G = 3, 64, 3000, 4                   # 48000 values per group: 2 slices
    y = torch.randn(N, C, L, generator=g) * 3 - 1
    assert c1g.load_library().c1g_gn_stats_workspace_size(N, C, L, G) > 0
    yd = to_dev(y)
    m1, r1 = c1g.gn_stats(yd, G)
    m2, r2 = c1g.gn_stats(yd, G)
    assert torch.equal(m1, m2) and torch.equal(r1, r2)
    flat = torch.empty(N * C * L + 1, device=DEV)
    yo = flat[1:].view(N, C, L)
    yo.copy_(yd)
    assert yo.data_ptr() % 16 == 4
    m3, r3 = c1g.gn_stats(yo, G)
    _, m_ref, r_ref = oracle.group_norm(y.double().numpy(), G, 1e-5)
    for m, r in ((m1, r1), (m3, r3)):
        assert max_abs_err(m, m_ref) <= 1e-5
        assert float(np.max(np.abs(r.cpu().double().numpy() / r_ref - 1))) <= 1e-5


def test_error_status_no_launch():
    """Invalid calls return a status and leave the output untouched."""
    announce("errors")
    x = torch.randn(2, 4, 50, device=DEV)
    w = torch.randn(8, 4, 3, device=DEV)
    out = torch.full((2, 8, 48), 7.0, device=DEV)
    with pytest.raises(c1g.C1GError) as ei:
        c1g.conv1d_gn_forward(x, w, norm="group", groups=3, out=out)   # 8 % 3 != 0
    assert ei.value.status == 1
    # a workspace that is not 256-byte aligned: C1G_ERR_MISALIGNED, nothing launched
    xb, wb = x.to(torch.bfloat16), w.to(torch.bfloat16)
    need = c1g.conv1d_gn_workspace_size(
        c1g.make_desc(2, 4, 8, 50, 3, dtype=c1g.C1G_BF16), c1g.make_norm("group", 2))
    assert need > 0
    ws = torch.empty(need + 256, device=DEV, dtype=torch.uint8)[16:]
    with pytest.raises(c1g.C1GError) as ei:
        c1g.conv1d_gn_forward(xb, wb, norm="group", groups=2, out=out, workspace=ws)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 7.0))


@pytest.mark.parametrize("wl", [GN_CASES[1], GN_CASES[-1]], ids=lambda w: w.name)
def test_groupnorm_invariant_on_device(wl):
    """With unit affine, every (n, group) of the output has mean 0 and variance
    var / (var + eps), where var = 1 / rstd^2 - eps is the group's variance the
    library itself reports: a property of the device result alone."""
    announce("GN invariant", wl.name)
    inp = make_inputs(wl.replace(affine=False), 3)
    out, mean, rstd = run_library(wl.replace(affine=False), inp, return_stats=True)
    z = out.double().cpu().numpy()
    N, C, T = z.shape
    zg = z.reshape(N, wl.G, (C // wl.G) * T)
    r = rstd.double().cpu().numpy()
    assert float(np.abs(zg.mean(axis=2)).max()) <= 1e-5
    want = 1.0 - wl.eps * r * r
    assert float(np.abs(zg.var(axis=2) / want - 1).max()) <= 1e-4


# N = 0: every entry point returns an empty result without launching anything
EMPTY_CASES = [
    dict(name="fused_fp32", C_in=16, C_out=32, T=256, K=3, pad=1, dil=1, dtype=torch.float32,
         norm="group", G=8, rowmin=False),
    dict(name="persistent_bf16", C_in=64, C_out=128, T=512, K=5, pad=4, dil=2,
         dtype=torch.bfloat16, norm="layer_channels", G=0, rowmin=False),
    dict(name="gemm_bf16", C_in=256, C_out=512, T=1, K=1, pad=0, dil=1, dtype=torch.bfloat16,
         norm="group", G=32, rowmin=True),
]


@pytest.mark.parametrize("case", EMPTY_CASES, ids=lambda c: c["name"])
def test_empty_batch(case):
    announce("empty batch", case["name"])
    C_in, C_out, T, K = case["C_in"], case["C_out"], case["T"], case["K"]
    dt = case["dtype"]
    x = torch.empty((0, C_in, T), device=DEV, dtype=dt)
    w = torch.randn((C_out, C_in, K), device=DEV).to(dt)
    b = torch.randn((C_out,), device=DEV)
    b2 = torch.randn((C_out,), device=DEV) if case["rowmin"] else None
    kw = dict(pad_left=case["pad"], pad_right=case["pad"], dilation=case["dil"])
    T_out = T + 2 * case["pad"] - case["dil"] * (K - 1)
    out, mean, rstd = c1g.conv1d_gn_forward(x, w, b, norm=case["norm"], groups=case["G"],
                                            rowmin_bias=b2, return_stats=True, **kw)
    assert out.shape == (0, C_out, T_out)
    assert mean.shape[0] == 0 and rstd.shape[0] == 0
    y = c1g.conv1d_forward(x, w, b, **kw)
    assert y.shape == (0, C_out, T_out)
    if case["norm"] == "group" and not case["rowmin"]:
        o2 = torch.empty((0, C_out, T_out), device=DEV)
        c1g.conv1d_gn_forward_noalloc(x, w, b, out=o2, norm="group", groups=case["G"], **kw)
    torch.cuda.synchronize()


def test_empty_batch_passes():
    announce("empty batch: gn_stats / gn_apply")
    y = torch.empty((0, 64, 100), device=DEV)
    mean, rstd = c1g.gn_stats(y, 8)
    assert mean.shape == (0, 8) and rstd.shape == (0, 8)
    out = c1g.gn_apply(y, mean, rstd, groups=8)
    assert out.shape == (0, 64, 100)
    yb = y.to(torch.bfloat16)
    assert c1g.gn_apply(yb, mean, rstd, groups=8).shape == (0, 64, 100)
    torch.cuda.synchronize()


# x one element past a 16-byte boundary: the kernels' unaligned staging paths
# (register-staged fused kernel, element-wise window loads, scalar input pack)
UNALIGNED_CASES = [
    Workload("unaligned_fused_fp32", N=2, C_in=32, C_out=64, T=300, K=3, pad_left=1,
             pad_right=1, G=8),
    Workload("unaligned_split_fp32", N=2, C_in=24, C_out=40, T=1500, K=5, dilation=2,
             pad_left=4, G=5),
    Workload("unaligned_bf16_persistent", N=2, C_in=40, C_out=128, T=600, K=5, dilation=2,
             pad_left=2, pad_right=2, G=8, dtype="bf16"),
    Workload("unaligned_bf16_split_ln", N=2, C_in=40, C_out=96, T=333, K=3, pad_left=1,
             pad_right=1, norm="layer_channels", dtype="bf16", persistent=False),
]


@pytest.mark.parametrize("wl", UNALIGNED_CASES, ids=lambda w: w.name)
def test_unaligned_x_matches_aligned(wl):
    """The same values handed over at an address one element past a 16-byte
    boundary give the same bits as from an aligned address."""
    announce("unaligned x", wl.name)
    inp = make_inputs(wl, 9)
    x = to_dev(inp["x"])
    flat = torch.empty(x.numel() + 1, device=DEV, dtype=x.dtype)
    xo = flat[1:].view(x.shape)
    xo.copy_(x)
    assert xo.data_ptr() % 16 != 0
    w = to_dev(inp["w"])
    kw = dict(stride=wl.stride, dilation=wl.dilation, pad_left=wl.pad_left,
              pad_right=wl.pad_right, norm=wl.norm, groups=wl.G, eps=wl.eps,
              gamma=to_dev(inp["gamma"]), beta=to_dev(inp["beta"]), persistent=wl.persistent)
    a = c1g.conv1d_gn_forward(x, w, to_dev(inp["bias"]), **kw)
    b = c1g.conv1d_gn_forward(xo, w, to_dev(inp["bias"]), **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, b)


def test_unaligned_x_on_the_gemm_route_is_rejected():
    """The Linear route copies 16-byte pieces of x and w: an unaligned x is a
    status (misaligned), reported before any launch."""
    announce("unaligned x, gemm route")
    x = torch.randn(33 * 64 + 1, device=DEV).to(torch.bfloat16)[1:].view(33, 64, 1)
    w = torch.randn(128, 64, 1, device=DEV).to(torch.bfloat16)
    with pytest.raises(c1g.C1GError) as e:
        c1g.conv1d_gn_forward(x, w, None, norm="group", groups=8)
    assert e.value.status == 4


def test_caller_workspace():
    """A caller's workspace may have any dtype: enough bytes give the bits of
    the library-allocated one.  One in host memory, or short of the size
    query in bytes, is refused before anything runs."""
    wl = Workload("ws_split_f32", N=2, C_in=24, C_out=48, T=1500, K=3, pad_left=1, pad_right=1,
                  G=6)
    announce("caller workspace", wl.name)
    inp = make_inputs(wl, 5)
    x, w, b, ga, be = (inp[k].to(DEV) for k in ("x", "w", "bias", "gamma", "beta"))
    kw = dict(pad_left=1, pad_right=1, norm="group", groups=6, gamma=ga, beta=be)
    ref = c1g.conv1d_gn_forward(x, w, b, **kw)
    need = c1g.conv1d_gn_workspace_size(
        c1g.make_desc(2, 24, 48, 1500, 3, pad_left=1, pad_right=1),
        c1g.make_norm("group", 6))
    assert need > 0
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=DEV)
    got = c1g.conv1d_gn_forward(x, w, b, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    with pytest.raises(ValueError, match="workspace"):
        c1g.conv1d_gn_forward(x, w, b, workspace=torch.empty(need, dtype=torch.uint8), **kw)
    with pytest.raises(c1g.C1GError, match="workspace"):
        c1g.conv1d_gn_forward(x, w, b, workspace=torch.empty(need // 8, dtype=torch.float32,
                                                             device=DEV), **kw)
