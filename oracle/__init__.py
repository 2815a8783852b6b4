"""fp64 CPU oracle for the conv1d -> GroupNorm path.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``conv1d_implicit_gemm_amd``) never imports this package, and this package
never imports the product: they share no code.  Only the seeded input
generator (``conv1d_implicit_gemm_amd.workloads``, which holds none of the
method's arithmetic) feeds both.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential sums,
OpenMP over independent outputs).  This module only builds it with gcc and
marshals numpy arrays.  Each function cites the passage of the pages it
follows; ``oracle.c`` writes the definitions out.

Functions: ``out_len``, ``conv1d``, ``group_norm``, ``layer_norm_channels``,
``rowmin_bias`` and ``forward`` (the composition the library's
``conv1d_gn_forward`` computes).  All are pinned by ``tests/test_oracle_*.py``
against closed forms, the pages' worked example, invariants, an independent
brute-force implementation and float64 library routines; the same pins are
run against deliberately broken copies of ``oracle.c`` to show they bite.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
_lock = threading.Lock()

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp, no fast-math, no contraction: the oracle's build line."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/_build/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(SOURCE, _LIB_PATH)
    return _LIB_PATH


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


class Oracle:
    """One loaded build of the oracle's C source."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_out_len.restype = _I64
        lib.oracle_out_len.argtypes = [_I64] * 6
        lib.oracle_conv1d.restype = None
        lib.oracle_conv1d.argtypes = [_I64] * 9 + [_D, _D, _D, _D]
        lib.oracle_group_norm.restype = None
        lib.oracle_group_norm.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_double,
                                          _D, _D, _D, _D, _D, _D]
        lib.oracle_layer_norm_channels.restype = None
        lib.oracle_layer_norm_channels.argtypes = [_I64, _I64, _I64, ctypes.c_double,
                                                   _D, _D, _D, _D, _D, _D]
        lib.oracle_rowmin_bias.restype = None
        lib.oracle_rowmin_bias.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D]
        self.lib = lib
        self.path = lib_path

    def num_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Set the OpenMP thread count of the following calls (n >= 1)."""
        self.lib.oracle_set_num_threads(int(n))

    def out_len(self, T, K, stride=1, dilation=1, pad_left=0, pad_right=0) -> int:
        """T_out = floor((T + pad_left + pad_right - dilation*(K-1) - 1)/stride) + 1, or -1.

        "Kimi-K2.6 l2_p35", T_out derivation for the default configuration
        (symmetric padding p is pad_left = pad_right = p); causal padding per
        "Kimi-K2.6 l1_p5" is pad_left = (K-1)*dilation, pad_right = 0.
        """
        return int(self.lib.oracle_out_len(T, K, stride, dilation, pad_left, pad_right))

    def conv1d(self, x, w, bias=None, stride=1, dilation=1, pad_left=0, pad_right=0):
        """Direct cross-correlation in fp64 ("Kimi-K2.6 l2_p35" conv index
        rule; "Kimi-K2.6 l1_p5" causal index rule).  x [N,C_in,T],
        w [C_out,C_in,K], bias [C_out] or None -> y [N,C_out,T_out]."""
        x, w, bias = _f64(x), _f64(w), _f64(bias)
        N, C_in, T = x.shape
        C_out, C_in_w, K = w.shape
        if C_in_w != C_in:
            raise ValueError("w and x disagree on C_in")
        T_out = self.out_len(T, K, stride, dilation, pad_left, pad_right)
        if T_out < 1:
            raise ValueError("no valid output length")
        if bias is not None and bias.shape != (C_out,):
            raise ValueError("bias must be [C_out]")
        y = np.empty((N, C_out, T_out), dtype=np.float64)
        self.lib.oracle_conv1d(N, C_in, C_out, T, K, stride, dilation, pad_left, pad_right,
                               _ptr(x), _ptr(w), _ptr(bias), _ptr(y))
        return y

    def group_norm(self, y, G, eps=1e-5, gamma=None, beta=None):
        """GroupNorm over (C/G channels x L) per (n, group), population
        variance, eps inside the root, per-channel affine ("Kimi-K2.6
        l2_p35", GroupNorm definition and population-variance check).
        Returns (z, mean[N,G], rstd[N,G])."""
        y, gamma, beta = _f64(y), _f64(gamma), _f64(beta)
        N, C, L = y.shape
        if G < 1 or C % G:
            raise ValueError("C must be a multiple of G")
        z = np.empty_like(y)
        mean = np.empty((N, G))
        rstd = np.empty((N, G))
        self.lib.oracle_group_norm(N, C, L, G, float(eps), _ptr(y), _ptr(gamma), _ptr(beta),
                                   _ptr(z), _ptr(mean), _ptr(rstd))
        return z, mean, rstd

    def layer_norm_channels(self, y, eps=1e-5, gamma=None, beta=None):
        """LayerNorm of the C values at every (n,l) with per-channel affine.
        Returns (z, mean[N,L], rstd[N,L])."""
        y, gamma, beta = _f64(y), _f64(gamma), _f64(beta)
        N, C, L = y.shape
        z = np.empty_like(y)
        mean = np.empty((N, L))
        rstd = np.empty((N, L))
        self.lib.oracle_layer_norm_channels(N, C, L, float(eps), _ptr(y), _ptr(gamma),
                                            _ptr(beta), _ptr(z), _ptr(mean), _ptr(rstd))
        return z, mean, rstd

    def rowmin_bias(self, z, bias2):
        """out[n,c,l] = min_c' z[n,c',l] + bias2[c] ("Kimi-K2.6 l2_p75",
        min over channels then broadcast bias).  Returns (out, rowmin[N,L])."""
        z, bias2 = _f64(z), _f64(bias2)
        N, C, L = z.shape
        out = np.empty_like(z)
        m = np.empty((N, L))
        self.lib.oracle_rowmin_bias(N, C, L, _ptr(z), _ptr(bias2), _ptr(out), _ptr(m))
        return out, m

    def forward(self, x, w, bias=None, *, stride=1, dilation=1, pad_left=0, pad_right=0,
                norm="group", G=1, eps=1e-5, gamma=None, beta=None, bias2=None):
        """The whole path: conv -> (GroupNorm | LayerNorm over channels | none)
        -> optional row-min + bias2.  Returns dict(out, y, mean, rstd, rowmin)."""
        y = self.conv1d(x, w, bias, stride, dilation, pad_left, pad_right)
        res = {"y": y, "mean": None, "rstd": None, "rowmin": None}
        if norm == "group":
            z, res["mean"], res["rstd"] = self.group_norm(y, G, eps, gamma, beta)
        elif norm == "layer_channels":
            z, res["mean"], res["rstd"] = self.layer_norm_channels(y, eps, gamma, beta)
        elif norm is None or norm == "none":
            z = y
        else:
            raise ValueError("unknown norm %r" % (norm,))
        if bias2 is not None:
            z, res["rowmin"] = self.rowmin_bias(z, bias2)
        res["out"] = z
        return res


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (rebuilt when the source is newer)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(SOURCE)):
                build(force=True)
            _default = Oracle(_LIB_PATH)
        return _default


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    return default().set_num_threads(n)


def out_len(*a, **k):
    return default().out_len(*a, **k)


def conv1d(*a, **k):
    return default().conv1d(*a, **k)


def group_norm(*a, **k):
    return default().group_norm(*a, **k)


def layer_norm_channels(*a, **k):
    return default().layer_norm_channels(*a, **k)


def rowmin_bias(*a, **k):
    return default().rowmin_bias(*a, **k)


def forward(*a, **k):
    return default().forward(*a, **k)
