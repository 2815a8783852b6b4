"""The library's environment switches on the GPU.  C1G_FORCE_PATH=split runs
problems planned on a single-kernel route (fused_single_pass,
fused_persistent) down the split route: both agree with the oracle, and with
each other to the tolerance.  C1G_LOG=1 reports each call's route, and a
fallback taken at run time (fewer resident workgroups than the plan needs,
forced with C1G_RESIDENT_LIMIT) with its cause."""
import pytest

from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import (TOL_BF16, TOL_F32, announce, check_parity, library_route,
                            max_abs_err, run_library)

pytestmark = pytest.mark.gpu

BF = dict(dtype="bf16")
FORCE_CASES = [
    (Workload("force_fused_f32", N=3, C_in=40, C_out=64, T=700, K=3, pad_left=1, pad_right=1,
              G=8), "fused_single_pass"),
    (Workload("force_persistent_gn", N=4, C_in=64, C_out=256, T=1100, K=5, dilation=2,
              pad_left=4, pad_right=4, G=16, **BF), "fused_persistent"),
    (Workload("force_persistent_ln", N=3, C_in=40, C_out=272, T=700, K=3, pad_left=1,
              pad_right=1, norm="layer_channels", **BF), "fused_persistent"),
]


@pytest.mark.parametrize("wl,route", FORCE_CASES, ids=[c[0].name for c in FORCE_CASES])
def test_force_split_agrees(wl, route, monkeypatch):
    assert library_route(wl) == route
    inp = make_inputs(wl, 13)
    default = run_library(wl, inp)
    monkeypatch.setenv("C1G_FORCE_PATH", "split")
    assert library_route(wl) == "split"
    check_parity(wl, seed=13)
    forced = run_library(wl, inp)
    monkeypatch.delenv("C1G_FORCE_PATH")
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_F32
    assert max_abs_err(forced, default.double().cpu().numpy()) <= tol


def test_log_reports_route_and_fallbacks(monkeypatch, capfd):
    wl = FORCE_CASES[1][0]
    gemm = Workload("log_gemm_one_launch", N=300, C_in=256, C_out=512, T=1, K=1, G=32,
                    rowmin_bias=True, one_launch=True, **BF)
    announce("C1G_LOG", wl.name, gemm.name)
    monkeypatch.setenv("C1G_LOG", "1")
    inp = make_inputs(wl, 3)
    ginp = make_inputs(gemm, 3)
    capfd.readouterr()
    run_library(wl, inp)
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("c1g: ")]
    assert len(lines) == 1 and "| fused_persistent T_out=1100 tiles=3x2" in lines[0]
    assert lines[0].endswith("-> ok"), lines[0]
    monkeypatch.setenv("C1G_RESIDENT_LIMIT", "1")
    run_library(wl, inp)
    run_library(gemm, ginp)
    monkeypatch.delenv("C1G_RESIDENT_LIMIT")
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("c1g: ")]
    assert len(lines) == 2, lines
    assert lines[0].endswith("the split route ran"), lines[0]
    assert "| gemm_rows" in lines[1] and lines[1].endswith("two launches"), lines[1]
