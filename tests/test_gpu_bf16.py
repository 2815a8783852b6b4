"""GPU parity of the bf16 path (bf16 x and w, fp32 accumulation and outputs)
against the fp64 oracle on the same bf16 values: max-abs 2e-2 after
normalisation, element by element."""
import numpy as np
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
from conv1d_implicit_gemm_amd.workloads import GENERALITY, WORKLOADS, Workload, make_inputs
from tests.gpu_util import (TOL_BF16, announce, check_parity, max_abs_err, run_library,
                            run_oracle)

pytestmark = pytest.mark.gpu

W = Workload
BF = dict(dtype="bf16")
# conv tiles: 512 (or 128 for wide windows) positions x 128 channels, 32 input
# channels per chunk; shapes span several tiles and end in ragged tails
CONV_CASES = [
    W("bf16_conv_gn_k5d2_3tiles", N=2, C_in=72, C_out=160, T=1300, K=5, dilation=2,
      pad_left=2, pad_right=2, G=8, **BF),
    W("bf16_conv_ln_3tiles", N=1, C_in=40, C_out=272, T=1300, K=5, dilation=2, pad_left=2,
      pad_right=2, norm="layer_channels", **BF),
    W("bf16_conv_gn_k5d2", N=2, C_in=72, C_out=160, T=300, K=5, dilation=2, pad_left=2,
      pad_right=2, G=8, **BF),
    W("bf16_conv_gn_causal", N=2, C_in=64, C_out=96, T=264, K=4, pad_left=3, G=12, **BF),
    W("bf16_conv_gn_odd_T", N=2, C_in=40, C_out=64, T=203, K=3, pad_left=1, pad_right=1,
      G=4, **BF),
    W("bf16_conv_gn_stride3_small_tile", N=2, C_in=33, C_out=48, T=401, K=3, stride=3,
      pad_left=1, pad_right=1, G=6, **BF),
    W("bf16_conv_only", N=3, C_in=48, C_out=130, T=256, K=2, norm=None, **BF),
    W("bf16_conv_ln", N=2, C_in=64, C_out=200, T=140, K=5, dilation=2, pad_left=2,
      pad_right=2, norm="layer_channels", **BF),
    W("bf16_conv_gn_rowmin", N=2, C_in=32, C_out=64, T=96, K=3, pad_left=1, pad_right=1,
      G=4, rowmin_bias=True, **BF),
    # 6..8 taps: 128-position tiles with an 8-tap weight stage
    W("bf16_conv_gn_k8", N=2, C_in=48, C_out=144, T=300, K=8, pad_left=3, pad_right=4,
      G=9, **BF),
    W("bf16_conv_gn_k7d2_causal", N=2, C_in=40, C_out=64, T=270, K=7, dilation=2,
      pad_left=12, G=8, **BF),
    W("bf16_conv_ln_k6", N=1, C_in=64, C_out=130, T=200, K=6, pad_left=2, pad_right=3,
      norm="layer_channels", **BF),
    # the widest windows: 8 taps at dilation 13 (219 of 224 rows on a
    # 128-position tile); 5 taps at dilation 9 (too wide for 512 positions)
    W("bf16_conv_gn_k8d13_widest", N=1, C_in=40, C_out=64, T=300, K=8, dilation=13,
      pad_left=45, pad_right=46, G=4, **BF),
    W("bf16_conv_gn_k5d9_small_tile", N=1, C_in=32, C_out=128, T=700, K=5, dilation=9,
      pad_left=18, pad_right=18, G=8, **BF),
]


@pytest.mark.parametrize("wl", CONV_CASES, ids=lambda w: w.name)
def test_bf16_conv_parity(wl):
    check_parity(wl)


# LayerNorm over channels on the split route: the apply pass that walks the
# channels of four positions (T_out % 4 == 0; a channel count that is no
# multiple of its 32-channel blocks; fp32 and bf16 out) and the general one
# (T_out % 4 != 0)
LN_SPLIT_CASES = [
    W("ln_split_cols_f32out", N=3, C_in=48, C_out=200, T=1032, K=5, dilation=2, pad_left=2,
      pad_right=2, norm="layer_channels", persistent=False, **BF),
    W("ln_split_cols_bf16out", N=2, C_in=40, C_out=70, T=520, K=3, pad_left=1, pad_right=1,
      norm="layer_channels", persistent=False, out_dtype="bf16", **BF),
    W("ln_split_general_T_out_odd", N=2, C_in=40, C_out=96, T=523, K=3, pad_left=1,
      pad_right=1, norm="layer_channels", persistent=False, **BF),
]


@pytest.mark.parametrize("wl", LN_SPLIT_CASES, ids=lambda w: w.name)
def test_ln_split_parity(wl):
    from tests.gpu_util import library_route
    assert library_route(wl) == "split"
    check_parity(wl)


# K = 1, T = 1: the GEMM route, with every epilogue combination
GEMM_CASES = [
    W("gemm_gn_rowmin_fused", N=70, C_in=256, C_out=512, T=1, K=1, G=32, bias=False,
      rowmin_bias=True, **BF),
    W("gemm_gn_rowmin_ragged", N=130, C_in=136, C_out=272, T=1, K=1, G=17, rowmin_bias=True,
      **BF),
    W("gemm_gn_rowmin_cpg8", N=40, C_in=64, C_out=256, T=1, K=1, G=32, rowmin_bias=True, **BF),
    W("gemm_gn", N=33, C_in=96, C_out=128, T=1, K=1, G=8, **BF),
    W("gemm_ln", N=33, C_in=96, C_out=200, T=1, K=1, norm="layer_channels", **BF),
    W("gemm_only", N=50, C_in=64, C_out=300, T=1, K=1, norm=None, **BF),
    W("gemm_rowmin_only", N=20, C_in=64, C_out=48, T=1, K=1, norm=None, rowmin_bias=True, **BF),
    # reduction shorter than one 64-wide chunk (tail only)
    W("gemm_tail_only", N=17, C_in=40, C_out=64, T=1, K=1, G=4, rowmin_bias=True, **BF),
    # odd number of whole chunks plus a tail
    W("gemm_odd_chunks_tail", N=90, C_in=200, C_out=128, T=1, K=1, G=8, **BF),
    # GroupNorm + row-min in one launch over 3 row blocks x 5
    # channel tiles, both ragged (1040 = 4 * 256 + 16 channels, 300 = 2 * 128 + 44
    # rows), and the same as a GEMM plus a broadcast kernel
    W("gemm_gn_rowmin_one_launch_ragged", N=300, C_in=200, C_out=1040, T=1, K=1, G=65,
      rowmin_bias=True, one_launch=True, **BF),
    W("gemm_gn_rowmin_two_launch_ragged", N=300, C_in=200, C_out=1040, T=1, K=1, G=65,
      rowmin_bias=True, **BF),
]


@pytest.mark.parametrize("wl", GEMM_CASES, ids=lambda w: w.name)
def test_bf16_gemm_parity(wl):
    check_parity(wl)


def test_gemm_route_is_taken():
    d = c1g.make_desc(1024, 8192, 8192, 1, 1, dtype=c1g.C1G_BF16)
    assert c1g.route(d, c1g.make_norm("group", 512, 1e-5, True)) == "gemm_rows"


@pytest.mark.parametrize("name", ["gemm_gn_rowmin_one_launch_ragged",
                                  "gemm_gn_rowmin_bf16_m1024_n8192_k8192"])
def test_gemm_rowmin_one_and_two_launches_identical(name):
    """GroupNorm + row-min + bias2 as one cooperative launch and as a GEMM plus
    a broadcast kernel: the same arithmetic in the same order, and a minimum is
    exact, so the outputs and statistics agree bit for bit."""
    wl = WORKLOADS.get(name) or next(w for w in GEMM_CASES if w.name == name)
    announce("gemm one vs two launches", wl.name)
    inp = make_inputs(wl, 3)
    one = run_library(wl.replace(one_launch=True), inp, return_stats=True)
    two = run_library(wl.replace(one_launch=False), inp, return_stats=True)
    for a, b in zip(one, two):
        assert torch.equal(a, b)


def test_linear_gn_rowmin_full_size_sampled():
    """The Linear -> GroupNorm -> min -> +bias workload at full size; the
    oracle checks 12 whole rows (every row's result depends on that row only)."""
    wl = WORKLOADS["gemm_gn_rowmin_bf16_m1024_n8192_k8192"]
    announce(wl.name)
    inp = make_inputs(wl, 0)
    got = run_library(wl, inp)
    rows = [0, 1, 2, 127, 128, 255, 256, 511, 640, 1000, 1022, 1023]
    ref = run_oracle(wl, inp, n_slice=rows)
    err = max_abs_err(got[rows], ref["out"])
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("name", ["conv1d_gn_bf16_n64_c512x1024_t4096_k5d2",
                                  "conv1d_lnc_bf16_n64_c512x1024_t4096_k5d2"])
def test_dilated_conv_full_size_sampled(name):
    """The bf16 dilated-conv workload at full size; the oracle checks two whole
    samples (GroupNorm and channel-LayerNorm statistics are per sample)."""
    wl = WORKLOADS[name]
    announce(wl.name)
    inp = make_inputs(wl, 0)
    got = run_library(wl, inp)
    for n in (0, wl.N - 1):
        ref = run_oracle(wl, inp, n_slice=slice(n, n + 1))
        err = max_abs_err(got[n:n + 1], ref["out"])
        assert err <= TOL_BF16, (n, err)


def test_bf16_determinism():
    wl = CONV_CASES[0]
    announce("bf16 determinism")
    inp = make_inputs(wl, 4)
    assert torch.equal(run_library(wl, inp), run_library(wl, inp))
    g = GEMM_CASES[0]
    inp = make_inputs(g, 4)
    assert torch.equal(run_library(g, inp), run_library(g, inp))


# The persistent route: one launch in rounds of whole samples
# (256 resident workgroups / tiles per sample = samples per round), partial
# statistics published, merged after a barrier among the sample's workgroups,
# the output written once.
PERSIST_CASES = [
    # 5 x 4 tiles per sample -> 12 samples per round: two rounds, the second partial
    W("persist_gn_2rounds", N=14, C_in=64, C_out=512, T=2200, K=3, pad_left=1, pad_right=1,
      G=32, **BF),
    W("persist_ln_2rounds", N=14, C_in=64, C_out=512, T=2200, K=3, pad_left=1, pad_right=1,
      norm="layer_channels", **BF),
    # one group spans two channel tiles (C_out/G = 256)
    W("persist_gn_group_spans_tiles", N=3, C_in=40, C_out=512, T=700, K=5, dilation=2,
      pad_left=4, pad_right=4, G=2, **BF),
    # a single group over all 256 channels (two channel tiles)
    W("persist_gn_g1", N=3, C_in=40, C_out=256, T=600, K=3, pad_left=1, pad_right=1, G=1,
      **BF),
    # one channel per group, ragged channel tile (200 = 128 + 72)
    W("persist_gn_cpg1_ragged", N=5, C_in=33, C_out=200, T=300, K=3, pad_left=1, pad_right=1,
      G=200, **BF),
    # 8 taps: 128-position tiles
    W("persist_ln_k8", N=4, C_in=48, C_out=144, T=300, K=8, pad_left=3, pad_right=4,
      norm="layer_channels", **BF),
    W("persist_gn_bf16_out", N=6, C_in=64, C_out=256, T=1100, K=5, dilation=2, pad_left=4,
      pad_right=4, G=16, out_dtype="bf16", **BF),
    # groups that straddle the 128-channel tiles: the whole sample waits, and
    # partials cover the largest power of two dividing the group width (<= 64)
    W("persist_gn_cpg48", N=3, C_in=40, C_out=192, T=1300, K=5, dilation=2, pad_left=4,
      pad_right=4, G=4, **BF),
    W("persist_gn_cpg24_ragged", N=4, C_in=33, C_out=240, T=700, K=3, pad_left=1,
      pad_right=1, G=10, **BF),
    W("persist_gn_cpg3", N=2, C_in=24, C_out=300, T=555, K=3, pad_left=1, pad_right=1, G=100,
      **BF),
    W("persist_gn_cpg96_stride2", N=3, C_in=64, C_out=384, T=1201, K=5, stride=2, pad_left=2,
      pad_right=2, G=4, **BF),
    W("persist_gn_cpg192", N=2, C_in=40, C_out=576, T=900, K=3, pad_left=1, pad_right=1, G=3,
      **BF),
    W("persist_gn_cpg80_k8_bf16out", N=3, C_in=48, C_out=160, T=450, K=8, pad_left=7, G=2,
      out_dtype="bf16", **BF),
    W("persist_gn_cpg48_k6", N=2, C_in=40, C_out=240, T=800, K=6, dilation=2, pad_left=10,
      G=5, **BF),
    # six and eight taps as two passes over the chunks on 512-position tiles:
    # four position tiles with a ragged last one, a partial last chunk,
    # straddling 25-channel groups; LayerNorm with a bf16 output
    W("persist_gn_k6_two_pass", N=5, C_in=72, C_out=200, T=1700, K=6, dilation=3, pad_left=7,
      pad_right=8, G=8, **BF),
    W("persist_ln_k8_two_pass_bf16out", N=3, C_in=40, C_out=136, T=1100, K=8, pad_left=7,
      norm="layer_channels", out_dtype="bf16", **BF),
    # seven taps: passes of four and three (the fourth slot's MFMAs skipped)
    W("persist_gn_k7_two_pass", N=3, C_in=72, C_out=192, T=1600, K=7, dilation=2, pad_left=6,
      pad_right=6, G=6, **BF),
]

# the same two-pass kernels on the split route
TWO_PASS_SPLIT = [
    W("split_gn_k8_two_pass", N=3, C_in=72, C_out=160, T=1300, K=8, pad_left=3, pad_right=4,
      G=5, persistent=False, **BF),
    W("split_ln_k6_two_pass", N=2, C_in=40, C_out=200, T=1111, K=6, dilation=2, pad_left=5,
      pad_right=5, norm="layer_channels", persistent=False, **BF),
    W("split_gn_k7_two_pass_bf16out", N=2, C_in=33, C_out=160, T=1234, K=7, pad_left=3,
      pad_right=3, G=8, out_dtype="bf16", persistent=False, **BF),
]


# strided convolutions as interleaved passes on 512-position tiles: one, two
# and three passes, passes with fewer taps than others (MFMAs skipped),
# dilation, channels-last input, bf16 output, straddling groups, the split
# and conv-only routes; several position tiles with a ragged last one
STRIDED_CASES = [
    (W("il_s2_k1_gn_cpg17", N=2, C_in=64, C_out=136, T=2100, K=1, stride=2, G=8, **BF),
     "fused_persistent"),
    (W("il_s2_k2_d3_ln", N=2, C_in=40, C_out=200, T=1999, K=2, stride=2, dilation=3,
       pad_left=1, pad_right=2, norm="layer_channels", **BF), "fused_persistent"),
    (W("il_s2_k4_causal_gn_bf16out", N=3, C_in=72, C_out=160, T=2400, K=4, stride=2,
       pad_left=3, G=4, out_dtype="bf16", **BF), "fused_persistent"),
    (W("il_s2_k7_d2_gn", N=2, C_in=40, C_out=144, T=2300, K=7, stride=2, dilation=2,
       pad_left=6, pad_right=6, G=9, **BF), "fused_persistent"),
    (W("il_s3_k2_gn_nlc", N=2, C_in=48, C_out=128, T=3100, K=2, stride=3, pad_left=1, G=16,
       channels_last=True, **BF), "fused_persistent"),
    (W("il_s3_k3_d2_gn", N=2, C_in=40, C_out=136, T=3300, K=3, stride=3, dilation=2,
       pad_left=2, pad_right=2, G=17, **BF), "fused_persistent"),
    (W("il_s3_k5_ln_split", N=2, C_in=33, C_out=150, T=3001, K=5, stride=3, pad_left=2,
       pad_right=2, norm="layer_channels", persistent=False, **BF), "split"),
    (W("il_s3_k8_causal_gn", N=2, C_in=40, C_out=128, T=2900, K=8, stride=3, pad_left=7, G=8,
       **BF), "fused_persistent"),
    (W("il_s2_k8_d4_conv_only", N=2, C_in=64, C_out=130, T=2500, K=8, stride=2, dilation=4,
       pad_left=14, norm=None, **BF), "conv_only"),
    # strides 4 and 5: four and five passes, one of them short
    (W("il_s4_k7_gn", N=2, C_in=40, C_out=136, T=4400, K=7, stride=4, pad_left=3, pad_right=3,
       G=8, **BF), "fused_persistent"),
    (W("il_s5_k5_ln_nlc", N=2, C_in=48, C_out=144, T=5200, K=5, stride=5, norm="layer_channels",
       channels_last=True, **BF), "fused_persistent"),
    (W("il_s5_k8_d2_gn_split_bf16out", N=2, C_in=33, C_out=128, T=5500, K=8, stride=5,
       dilation=2, pad_left=7, G=4, out_dtype="bf16", persistent=False, **BF), "split"),
]


@pytest.mark.parametrize("wl,route", STRIDED_CASES, ids=lambda c: getattr(c, "name", c))
def test_interleaved_strided_parity(wl, route):
    from tests.gpu_util import library_route
    assert library_route(wl) == route
    check_parity(wl)


@pytest.mark.parametrize("wl", TWO_PASS_SPLIT, ids=lambda w: w.name)
def test_two_pass_split_parity(wl):
    from tests.gpu_util import library_route
    assert library_route(wl) == "split"
    check_parity(wl)


@pytest.mark.parametrize("wl", PERSIST_CASES, ids=lambda w: w.name)
def test_persistent_route_parity(wl):
    from tests.gpu_util import library_route
    assert library_route(wl) == "fused_persistent"
    check_parity(wl)


def test_persistent_and_split_agree_with_oracle():
    """The same inputs through the persistent route and, with the persistent
    route switched off, the split route: both within tolerance of the oracle,
    statistics included."""
    wl = PERSIST_CASES[0]
    announce("persistent vs split", wl.name)
    inp = make_inputs(wl, 2)
    ref = run_oracle(wl, inp)
    x, w = (inp[k].to("cuda:0") for k in ("x", "w"))
    b, ga, be = (inp[k].to("cuda:0") for k in ("bias", "gamma", "beta"))
    for persistent in (True, False):
        out, mean, rstd = c1g.conv1d_gn_forward(x, w, b, pad_left=1, pad_right=1, norm="group",
                                                groups=wl.G, gamma=ga, beta=be,
                                                return_stats=True, persistent=persistent)
        torch.cuda.synchronize()
        assert max_abs_err(out, ref["out"]) <= TOL_BF16, persistent
        assert max_abs_err(mean, ref["mean"]) <= 1e-4, persistent
        r = rstd.cpu().double().numpy()
        assert float(np.max(np.abs(r / ref["rstd"] - 1))) <= 1e-4, persistent


@pytest.mark.parametrize("name", ["persist_gn_2rounds", "persist_ln_k8",
                                  "gemm_gn_rowmin_one_launch_ragged"])
def test_cooperative_launch_identical(name):
    """The kernels whose workgroups wait on each other give the same bits
    launched ordinarily (the default) and through the runtime's cooperative
    launch (C1G_FLAG_COOPERATIVE)."""
    wl = next(w for w in PERSIST_CASES + GEMM_CASES if w.name == name)
    announce("cooperative vs ordinary launch", wl.name)
    inp = make_inputs(wl, 3)
    plain = run_library(wl, inp, return_stats=True)
    coop = run_library(wl.replace(cooperative=True), inp, return_stats=True)
    for a, b in zip(plain, coop):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


def test_persistent_determinism():
    wl = PERSIST_CASES[1]
    announce("persistent determinism", wl.name)
    inp = make_inputs(wl, 5)
    assert torch.equal(run_library(wl, inp), run_library(wl, inp))


# Generality at scale: stride 2 to 4, 8 taps at dilation 2 and at stride 4, groups wider than 32
# channels (one group spanning channel tiles; groups of 48 that straddle the
# 128-channel tiles), channels-last input; the same
# workloads bench.py --mode generality times.  The oracle checks the first and
# the last sample of each.
SCALE_ROUTES = {"conv1d_gn_bf16_n32_c512x1024_t8192_k5s2": "fused_persistent",
                "conv1d_gn_bf16_n32_c512x1024_t16384_k8s4": "fused_persistent",
                "conv1d_gn_bf16_n32_c256x512_t4096_k8d2": "fused_persistent",
                "conv1d_lnc_bf16_n32_c512x512_t4096_k7": "fused_persistent",
                "conv1d_gn_bf16_n32_c512x1024_t4096_k5d2_g4": "fused_persistent",
                "conv1d_gn_bf16_n16_c256x1536_t4096_k3_g32": "fused_persistent",
                "conv1d_lnc_bf16_nlc_n30_c384x768_t6000_k4s3": "fused_persistent",
                "conv1d_gn_f32_n16_c256x256_t8192_k4s2": "split"}
assert set(SCALE_ROUTES) == set(GENERALITY)
SCALE_CASES = [(WORKLOADS[n], SCALE_ROUTES[n]) for n in GENERALITY]


@pytest.mark.parametrize("wl,route", SCALE_CASES, ids=lambda c: getattr(c, "name", c))
def test_generality_at_scale_sampled(wl, route):
    from tests.gpu_util import library_route, tol_for
    assert library_route(wl) == route
    announce("scale", wl.name)
    inp = make_inputs(wl, 0)
    got, mean, rstd = run_library(wl, inp, return_stats=True)
    for n in (0, wl.N - 1):
        ref = run_oracle(wl, inp, n_slice=slice(n, n + 1))
        err = max_abs_err(got[n:n + 1], ref["out"])
        assert err <= tol_for(wl), (n, err)
        assert max_abs_err(mean[n:n + 1], ref["mean"]) <= 1e-4
        r = rstd[n:n + 1].cpu().double().numpy()
        assert float(np.max(np.abs(r / ref["rstd"] - 1))) <= 1e-4


@pytest.mark.parametrize("which", ["persistent_conv", "gemm_one_launch"])
def test_barrier_give_up_poisons_output(which, monkeypatch):
    """A grid-barrier wait that gives up (forced from the host with
    C1G_BARRIER_SPINS=0: a workgroup that does not find its group complete at
    the first poll stops waiting) never hangs and never yields a plausible
    wrong value: the statistics of such a workgroup are NaN, so its output is
    NaN, while every finite output equals the normal result bit for bit.  The
    next call with the default limit is exact again."""
    if which == "persistent_conv":
        wl = PERSIST_CASES[0]
    else:
        wl = next(w for w in GEMM_CASES if w.name == "gemm_gn_rowmin_one_launch_ragged")
    announce("barrier give-up", wl.name)
    inp = make_inputs(wl, 7)
    ref = run_library(wl, inp, poison=False)
    monkeypatch.setenv("C1G_BARRIER_SPINS", "0")
    forced = run_library(wl, inp, poison=False)
    monkeypatch.delenv("C1G_BARRIER_SPINS")
    again = run_library(wl, inp, poison=False)
    assert torch.isfinite(ref).all() and torch.equal(again, ref)
    nan = torch.isnan(forced)
    assert nan.any(), "no workgroup gave up (the wait should fail at the first poll)"
    assert torch.equal(forced[~nan], ref[~nan])


# C1G_RESIDENT_LIMIT caps the resident workgroups the library assumes: the
# paths of a device that keeps fewer workgroups resident, on this one.
# PERSIST_CASES[0] and [1] have 5 x 4 = 20 tiles per sample (512 positions x
# 128 channels), so a cap of 20 gives one sample per round (14 rounds), 45
# two per round, and 19 too few for a sample: the split route runs instead.
RESIDENT_CASES = [(0, "20"), (0, "45"), (0, "19"), (1, "20"), (1, "19")]


@pytest.mark.parametrize("case,limit", RESIDENT_CASES,
                         ids=["%s_cap%s" % (PERSIST_CASES[c].name, l) for c, l in RESIDENT_CASES])
def test_resident_limit(case, limit, monkeypatch):
    """Fewer samples per round give the bits of the default rounds (each
    tile's arithmetic and each sample's merge order do not depend on the
    round), and a cap below one sample's tiles gives the bits of the split
    route (the same tiles and merge, the same workspace offsets); both stay
    within tolerance of the oracle on the first and last samples.  The
    planner still reports the persistent route: the choice is made per call."""
    from tests.gpu_util import library_route
    wl = PERSIST_CASES[case]
    announce("resident limit", limit, wl.name)
    inp = make_inputs(wl, 9)
    full = run_library(wl, inp)
    split = run_library(wl.replace(persistent=False), inp)
    monkeypatch.setenv("C1G_RESIDENT_LIMIT", limit)
    assert library_route(wl) == "fused_persistent"
    capped = run_library(wl, inp)
    monkeypatch.delenv("C1G_RESIDENT_LIMIT")
    assert torch.isfinite(capped).all()
    assert torch.equal(capped, split if int(limit) < 20 else full)
    for n in (0, wl.N - 1):
        ref = run_oracle(wl, inp, n_slice=slice(n, n + 1))
        assert max_abs_err(capped[n:n + 1], ref["out"]) <= TOL_BF16, n


def test_resident_limit_gemm_one_launch(monkeypatch):
    """The one-launch GEMM + row-min with a cap below its grid runs as the GEMM
    and a broadcast kernel: the same bits."""
    wl = next(w for w in GEMM_CASES if w.name == "gemm_gn_rowmin_one_launch_ragged")
    announce("resident limit", wl.name)
    inp = make_inputs(wl, 9)
    ref = run_library(wl, inp)
    monkeypatch.setenv("C1G_RESIDENT_LIMIT", "1")
    capped = run_library(wl, inp)
    monkeypatch.delenv("C1G_RESIDENT_LIMIT")
    assert torch.isfinite(ref).all() and torch.equal(capped, ref)
