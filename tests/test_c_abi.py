"""The C ABI from C.  On the CPU: include/conv1d_gn.h compiles as strict C99
and as C++, and tests/c_abi_consumer.c (a plain C caller: descriptors, route
and workspace queries, conv1d_gn_forward on its own HIP stream, an invalid
call refused with a status) compiles and links against the library, the
oracle and the HIP runtime.  On the GPU: that program runs and agrees with
the oracle."""
import os
import subprocess

import pytest

import conv1d_implicit_gemm_amd as c1g
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _consumer(tmp_path):
    """Compile and link the C consumer; returns the executable's path."""
    lib_dir = os.path.dirname(c1g.LIB_PATH)
    if not os.path.exists(c1g.LIB_PATH):
        pytest.fail("the library is not built: " + c1g.LIB_PATH)
    ora_dir = os.path.dirname(oracle.build(force=False))
    exe = str(tmp_path / "c_abi_consumer")
    rpath = ":".join([lib_dir, ora_dir, os.path.join(ROCM, "lib")])
    cmd = ["gcc", "-std=gnu99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", INCLUDE,
           os.path.join(HERE, "c_abi_consumer.c"), "-o", exe,
           "-L", lib_dir, "-lconv1d_gn", "-L", ora_dir, "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath," + rpath]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++11")])
def test_header_compiles_strictly(tmp_path, compiler, std):
    src = tmp_path / ("h.c" if compiler == "gcc" else "h.cpp")
    src.write_text('#include "conv1d_gn.h"\nint main(void) { return C1G_OK; }\n')
    cmd = [compiler, std, "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
           "-I", INCLUDE, str(src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_consumer_links(tmp_path):
    assert os.path.exists(_consumer(tmp_path))


@pytest.mark.gpu
def test_c_consumer_runs(tmp_path):
    exe = _consumer(tmp_path)
    print("running the C consumer", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
