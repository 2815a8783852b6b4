"""Property-based fuzzing of the host-side validation (CPU only).

Descriptors are drawn over the whole range of their C types, extremes
included, and handed to the planner directly (no Python-side checks):
  - c1g_check never fails outside the validation statuses, and whatever it
    accepts lies inside the documented limits (N up to 65535, C_in and C_out
    up to 2^30, T up to 2^40, x and w below 2^46 elements, N*C_out*T_out below
    2^32, valid enums, C_out % G == 0, finite eps > 0);
  - c1g_out_len matches the output-length formula in exact integers;
  - the workspace query is consistent with c1g_check (exactly that many bytes
    suffice, one fewer does not);
  - a call that gets as far as a launch attempt (status C1G_ERR_HIP, as there
    is no device here) lies inside the same limits; for gn_stats and gn_apply
    as well.  Those calls take fake, aligned addresses and run only where no
    GPU is present: validation reads no pointer, and the launch fails."""
import ctypes
import os

import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import conv1d_implicit_gemm_amd as c1g

# counting devices does not initialise one; either sign of a GPU skips the
# calls that take fake addresses
NO_GPU = not os.path.exists("/dev/kfd") and torch.cuda.device_count() == 0
FAKE = ctypes.c_void_p(1 << 24)
ROUTES = {"fused_single_pass", "fused_persistent", "gemm_rows", "split", "conv_only", "empty"}


I64_EDGES = [-1, 0, 1, 65535, 65536, 2 ** 30, 2 ** 30 + 1, 2 ** 31, 2 ** 32, 2 ** 40, 2 ** 40 + 1,
             2 ** 46, 2 ** 62, 2 ** 62 + 1, 2 ** 63 - 1, -2 ** 63]
I32_EDGES = [-1, 0, 1, 2, 3, 8, 9, 2 ** 15, 2 ** 30, 2 ** 31 - 1, -2 ** 31]
extreme64 = st.one_of(st.integers(-2 ** 63, 2 ** 63 - 1), st.sampled_from(I64_EDGES))
extreme32 = st.one_of(st.integers(-2 ** 31, 2 ** 31 - 1), st.sampled_from(I32_EDGES))
DESC64 = ("N", "C_in", "C_out", "T")
DESC32 = ("K", "stride", "dilation", "pad_left", "pad_right", "dtype", "out_dtype", "x_layout")
NORM32 = ("norm", "G", "epilogue", "flags")


@st.composite
def calls(draw):
    """A plausible descriptor pair, then 0-3 fields replaced by extreme values
    of their C type (or a non-finite / non-positive eps)."""
    C_out = draw(st.integers(1, 600))
    d = dict(N=draw(st.integers(0, 70)), C_in=draw(st.integers(1, 600)), C_out=C_out,
             T=draw(st.integers(1, 5000)), K=draw(st.integers(1, 10)),
             stride=draw(st.integers(1, 4)), dilation=draw(st.integers(1, 4)),
             pad_left=draw(st.integers(0, 10)), pad_right=draw(st.integers(0, 10)),
             dtype=draw(st.integers(0, 1)), out_dtype=draw(st.integers(0, 1)),
             x_layout=draw(st.integers(0, 1)))
    n = dict(norm=draw(st.integers(0, 2)),
             G=draw(st.sampled_from([g for g in range(1, 65) if C_out % g == 0])),
             eps=1e-5, epilogue=draw(st.integers(0, 1)), flags=draw(st.integers(0, 7)))
    kind = draw(st.sampled_from(["conv", "conv", "linear", "fused"]))
    if kind == "linear":  # K = 1, T = 1, C_in % 8 == 0: the gemm_rows route in bf16
        d.update(T=1, K=1, pad_left=0, pad_right=0, stride=1, dilation=1,
                 C_in=8 * draw(st.integers(1, 75)))
    elif kind == "fused":  # fp32 GroupNorm, C_out/G dividing 16, T_out up to 1024
        G = draw(st.integers(1, 32))
        d.update(dtype=0, T=draw(st.integers(1, 1024)), stride=1,
                 C_out=G * draw(st.sampled_from([1, 2, 4, 8, 16])))
        d["pad_right"] = d["pad_left"]
        n.update(norm=1, G=G, epilogue=0)
    for _ in range(draw(st.integers(0, 3))):
        f = draw(st.sampled_from(DESC64 + DESC32 + NORM32 + ("eps",)))
        if f in DESC64:
            d[f] = draw(extreme64)
        elif f in DESC32:
            d[f] = draw(extreme32)
        elif f == "eps":
            n[f] = draw(st.sampled_from([0.0, -1e-5, float("inf"), float("nan"), 1e-30]))
        else:
            n[f] = draw(extreme32)
    nd = c1g.NormDesc(**n) if draw(st.integers(0, 4)) else None
    return c1g.ConvDesc(**d), nd


def exact_out_len(d):
    span = d.T + d.pad_left + d.pad_right - d.dilation * (d.K - 1) - 1
    return span // d.stride + 1


def within_contract(d, nd):
    """The documented limits of conv1d_forward / conv1d_gn_forward."""
    if not (0 <= d.N <= 65535 and 1 <= d.C_in <= 2 ** 30 and 1 <= d.C_out <= 2 ** 30 and
            1 <= d.T <= 2 ** 40 and d.K >= 1 and d.stride >= 1 and d.dilation >= 1 and
            d.pad_left >= 0 and d.pad_right >= 0):
        return False
    if d.dtype not in (0, 1) or d.out_dtype not in (0, 1) or d.x_layout not in (0, 1):
        return False
    T_out = exact_out_len(d)
    if T_out < 1:
        return False
    if d.N > 0 and (d.N * d.C_out * T_out >= 2 ** 32 or d.N * d.C_in * d.T >= 2 ** 46 or
                    d.C_out * d.C_in * d.K >= 2 ** 46):
        return False
    if nd is not None:
        if nd.norm not in (0, 1, 2) or nd.epilogue not in (0, 1):
            return False
        if nd.norm == 1 and (nd.G < 1 or d.C_out % nd.G != 0):
            return False
        if nd.norm != 0 and not (nd.eps > 0 and nd.eps != float("inf")):
            return False
    return True


@settings(max_examples=3000, deadline=None, suppress_health_check=list(HealthCheck))
@given(call=calls())
def test_planner_accepts_only_the_contract(call):
    d, nd = call
    status = c1g.check(d, nd)
    assert status in (0, 1, 2, 3, 4)
    n = c1g.out_len(d)
    valid_geometry = (d.N >= 0 and d.C_in >= 1 and d.C_out >= 1 and 1 <= d.T <= 2 ** 62 and
                      d.K >= 1 and d.stride >= 1 and d.dilation >= 1 and d.pad_left >= 0 and
                      d.pad_right >= 0 and exact_out_len(d) >= 1)
    assert n == (exact_out_len(d) if valid_geometry else -1)
    r = c1g.route(d, nd)
    if status != 0:
        assert r == "invalid"
        return
    assert within_contract(d, nd), (status, r)
    assert r in ROUTES
    ws = (c1g.conv1d_gn_workspace_size(d, nd) if nd is not None
          else c1g.conv1d_workspace_size(d))
    assert ws < 2 ** 50 and ws % 256 == 0
    assert c1g.check(d, nd, ws) == 0
    if ws > 0:
        assert c1g.check(d, nd, ws - 1) == 3


@pytest.mark.skipif(not NO_GPU, reason="fake addresses are safe only where nothing can launch")
@settings(max_examples=1500, deadline=None, suppress_health_check=list(HealthCheck))
@given(call=calls())
def test_only_contract_calls_reach_a_launch(call):
    d, nd = call
    lib = c1g.load_library()
    F = FAKE
    if nd is None:
        status = lib.conv1d_forward(ctypes.byref(d), F, F, F, F, F, 1 << 62, None)
    else:
        status = lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(nd), F, F, F, F, F, F, F,
                                       None, None, F, 1 << 62, None)
    assert status in (0, 1, 2, 3, 4, 5)
    if status == 5:  # a launch was attempted
        assert within_contract(d, nd) and d.N > 0
    if status == 0:  # nothing to launch
        assert d.N == 0 and within_contract(d, nd)


@pytest.mark.skipif(not NO_GPU, reason="fake addresses are safe only where nothing can launch")
@settings(max_examples=1500, deadline=None, suppress_health_check=list(HealthCheck))
@given(N=st.one_of(st.integers(0, 64), extreme64), C=st.one_of(st.integers(1, 512), extreme64),
       L=st.one_of(st.integers(1, 5000), extreme64), G=st.one_of(st.integers(1, 64), extreme32))
def test_norm_passes_reach_a_launch_only_within_limits(N, C, L, G):
    lib = c1g.load_library()
    F = FAKE
    args_ok = N >= 0 and C >= 1 and L >= 1 and G >= 1 and C % G == 0
    s = lib.gn_apply(N, C, L, G, F, F, F, None, None, F, None)
    if s == 5:
        assert args_ok and N > 0 and C <= 2 ** 31 and L <= 2 ** 31 and N * C * L < 2 ** 32
    for_bf16 = lib.gn_apply_bf16(N, C, L, G, F, F, F, None, None, F, None)
    assert for_bf16 == s
    s = lib.gn_stats(N, C, L, G, 1e-5, F, F, F, F, 1 << 62, None)
    if s == 5:
        slices = ((C // G) * L + 32767) // 32768
        assert args_ok and N > 0 and N * G <= 2 ** 31 - 1 and N * G * slices <= 2 ** 31 - 1
    ws = lib.c1g_gn_stats_workspace_size(N, C, L, G)
    if not args_ok:
        assert ws == 0
