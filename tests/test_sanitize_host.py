"""The library's host code under the compiler's address and undefined-
behaviour checks (CPU only).  Every source is built with those checks on its
host side (-Xarch_host -fsanitize=address,undefined, no recovery: the first
finding stops the program) and linked with tests/sanitize_host.cpp, which
calls every host-side function of the C ABI with randomised and boundary
arguments: the planner, the size queries, the entry points' validation, the
log's formatting.  The program must finish without a finding.  Entry-point
calls take fake addresses, so the test runs only where no GPU is present:
there a call that passes validation fails at its launch and nothing runs."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "conv1d_implicit_gemm_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
NO_GPU = not os.path.exists("/dev/kfd") and torch.cuda.device_count() == 0
HOST_CHECKS = ["-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not NO_GPU, reason="fake addresses are safe only where nothing can launch")
def test_host_code_under_sanitizers(tmp_path):
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    base = [HIPCC, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", "-Xclang",
            "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_CHECKS + [
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run(base + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs + [os.path.join(HERE, "sanitize_host.cpp")]))
    exe = str(tmp_path / "sanitize_host")
    # the link takes the host runtimes only (no device code is instrumented)
    link = [HIPCC, "--offload-arch=gfx950", "-fno-gpu-sanitize", "-fsanitize=address,undefined"]
    r = subprocess.run(link + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, env=env, timeout=600)
    findings = [l for l in r.stderr.splitlines()
                if "Sanitizer" in l or "runtime error: " in l]
    assert r.returncode == 0 and r.stdout.startswith("OK "), (r.stdout, findings[:20])
    assert not findings, findings[:20]
