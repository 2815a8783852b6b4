"""bench.py's host-side contract (CPU only): the one-GPU refusal, the
FLOP and byte counts and roofline fractions it reports, the stored counter
record it reads only while the kernel source is unchanged, and the fields of
the oracle's CPU baseline."""
import json
import os
import re
import subprocess
import sys

import pytest

import bench
from conv1d_implicit_gemm_amd.workloads import HEADLINE, SMALL, WORKLOADS, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


class _Op:
    def __init__(self, T_out):
        self.T_out = T_out
        self.calls = 0

    def __call__(self):
        self.calls += 1


class _Timer:
    """Fixed timings in place of HIP events."""

    def flushed(self, op, reps):
        return 0.040, 0.035

    def warm(self, op, reps):
        return 0.0375


@pytest.mark.parametrize("name,T_out,flops,peak", [
    (HEADLINE, 1024, 2 * 16 * 1024 * 256 * 128 * 3, 157.3),
    ("causal_conv1d_f32_n32_c256x256_t8192_k4", 8192, 2 * 32 * 8192 * 256 * 256 * 4, 157.3),
    ("gemm_gn_rowmin_bf16_m1024_n8192_k8192", 1, 2 * 1024 * 8192 * 8192, 2500.0),
    ("conv1d_gn_bf16_n64_c512x1024_t4096_k5d2", 4092, 2 * 64 * 4092 * 1024 * 512 * 5, 2500.0),
])
def test_measure_counts_and_fractions(name, T_out, flops, peak):
    wl = WORKLOADS[name]
    op = _Op(T_out)
    m = bench.measure(wl, op, _Timer(), steps=20, warmup=5)
    assert op.calls == 5  # the warm-up steps; the stub timer runs none
    assert m["flops"] == flops
    assert m["peak"] == peak and m["bound"] == "mfma" and m["unit"] == "TFLOP/s"
    assert m["ms_median"] == 0.040 and m["ms_min"] == 0.035 and m["ms_warm"] == 0.0375
    assert m["tflops"] == pytest.approx(flops / 40e-6 / 1e12, rel=1e-12)
    assert m["frac"] == pytest.approx(m["tflops"] / peak, rel=1e-12)
    assert m["frac_warm"] == pytest.approx(flops / 37.5e-6 / 1e12 / peak, rel=1e-12)
    e = wl.elem_bytes
    assert m["algo_bytes"] == (wl.N * wl.C_in * wl.T * e + wl.C_out * wl.C_in * wl.K * e +
                               wl.N * wl.C_out * T_out * 4)


def _record(workload):
    txt = open(os.path.join(ROOT, "profiles", workload + ".md")).read()
    return json.loads(re.search(r"```json counters\n(.*?)\n```", txt, flags=re.S).group(1))


def test_stored_traffic_only_for_the_profiled_source(monkeypatch):
    rec = _record(HEADLINE)
    expect = (rec["hbm_bytes_per_launch"]
              if rec["kernel_source_sha256_16"] == bench.source_hash("fused_single_pass")
              else None)
    assert bench.stored_traffic(HEADLINE, "fused_single_pass") == expect
    # a route whose sources are not tracked, or a changed source: no figure
    assert bench.stored_traffic(HEADLINE, "split") is None
    monkeypatch.setattr(bench, "source_hash", lambda route: "0" * 16)
    assert bench.stored_traffic(HEADLINE, "fused_single_pass") is None
    assert bench.stored_traffic("no_such_workload", "fused_single_pass") is None


def test_cpu_baseline_fields():
    import oracle
    wl = WORKLOADS[SMALL]
    inp = make_inputs(wl, 0)
    flops = 2 * wl.N * 256 * wl.C_out * wl.C_in * wl.K
    cb = bench.cpu_baseline(wl, inp, flops, budget_s=0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["cores"] == oracle.num_threads() >= 1
    assert cb["value"] > 0 and "fp64" in cb["sample"]
    st = cb["single_thread"]
    assert st["cores"] == 1 and st["value"] > 0
    assert oracle.num_threads() == cb["cores"]  # the thread count is restored


def test_generality_workloads_plan_their_routes():
    """The full-scale cases bench.py --mode generality times take the routes
    their parity test expects (host planner only)."""
    from conv1d_implicit_gemm_amd.workloads import GENERALITY
    from tests.sweep_cases import route_of
    from tests.test_gpu_bf16 import SCALE_ROUTES
    assert tuple(SCALE_ROUTES) == GENERALITY
    for name in GENERALITY:
        assert route_of(WORKLOADS[name]) == SCALE_ROUTES[name], name
