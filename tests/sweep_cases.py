"""A seeded random sweep of small problems over everything the boundary
accepts: geometry (taps, stride, dilation, symmetric, asymmetric and causal
padding, ragged lengths), x and output dtypes, both input layouts, every
normalisation, the row-min epilogue and the persistent switch.

The cases are drawn once from a fixed seed, so a failing case is named and
reproducible; only cases the planner accepts (c1g_check == OK) are kept.
The drawing is plain host code (no device): the CPU suite checks that the
sweep reaches every route, the GPU suite runs each case against the oracle.
"""
import numpy as np

import conv1d_implicit_gemm_amd as c1g
from conv1d_implicit_gemm_amd.workloads import Workload

SWEEP_SEED = 20261202
SWEEP_SEEDS = tuple(SWEEP_SEED + k for k in range(8))  # independent draws
N_CASES = 96                                # per draw
MAX_MACS = 1.5e9  # keeps each oracle run under about a second


def _desc(wl: Workload):
    return c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K, stride=wl.stride,
                         dilation=wl.dilation, pad_left=wl.pad_left, pad_right=wl.pad_right,
                         dtype=c1g.C1G_BF16 if wl.dtype == "bf16" else c1g.C1G_F32,
                         out_dtype=c1g.C1G_BF16 if wl.out_dtype == "bf16" else c1g.C1G_F32,
                         x_layout=c1g.LAYOUT_NLC if wl.channels_last else c1g.LAYOUT_NCL)


def _norm(wl: Workload):
    return c1g.make_norm(wl.norm, wl.G, wl.eps, wl.rowmin_bias, wl.persistent, wl.one_launch)


def accepted(wl: Workload) -> bool:
    return c1g.check(_desc(wl), _norm(wl)) == 0


def route_of(wl: Workload) -> str:
    return c1g.route(_desc(wl), _norm(wl))


def _draw(rng, i, tag=""):
    dtype = str(rng.choice(["f32", "bf16"]))
    if rng.random() < 0.12:  # a Linear layer: K = 1, T = 1
        N = int(rng.integers(1, 200))
        C_in = 8 * int(rng.integers(1, 40))
        G = int(rng.choice([1, 2, 4, 8]))
        C_out = G * 8 * int(rng.integers(1, 6))
        return Workload("sweep%s%02d_linear" % (tag, i), N=N, C_in=C_in, C_out=C_out, T=1, K=1,
                        dtype="bf16", norm="group", G=G, rowmin_bias=bool(rng.random() < 0.7),
                        out_dtype=str(rng.choice(["f32", "bf16"])),
                        one_launch=bool(rng.random() < 0.3))
    norm = rng.choice(["none", "group", "group", "layer_channels"])
    norm = None if norm == "none" else str(norm)
    K = int(rng.integers(1, 9))
    d = int(rng.integers(1, 5)) if K > 1 else 1
    s = int(rng.choice([1, 1, 1, 1, 2, 3, 4, 5]))
    span = d * (K - 1)
    if rng.random() < 0.25:
        pl, pr = span, 0                                   # causal
    else:
        pl, pr = int(rng.integers(0, span + 2)), int(rng.integers(0, span + 2))
    big = rng.random() < 0.25                              # several tiles each way
    T = int(rng.integers(1, 5000 if big else 400))
    C_in = int(rng.integers(1, 600 if big else 72))
    if norm == "group":
        G = int(rng.integers(1, 17 if big else 9))
        C_out = G * int(rng.choice([1, 2, 4, 8, 16, 32]))
    else:
        G = 1
        C_out = int(rng.integers(1, 600 if big else 160))
    while T > 64 and 3 * C_out * T * C_in * K / s > MAX_MACS:
        T //= 2
    T = max(T, span + 1 - pl - pr)                         # at least one output
    return Workload(
        "sweep%s%02d_%s_%s_k%ds%dd%d" % (tag, i, dtype, norm or "conv", K, s, d),
        N=int(rng.integers(1, 4)), C_in=C_in, C_out=C_out, T=T, K=K, stride=s, dilation=d,
        pad_left=pl, pad_right=pr, dtype=dtype, norm=norm, G=G,
        out_dtype="bf16" if rng.random() < 0.25 else "f32",
        bias=bool(rng.random() < 0.8), affine=bool(rng.random() < 0.8),
        rowmin_bias=bool(norm is not None and rng.random() < 0.2),
        persistent=bool(rng.random() < 0.8), channels_last=bool(rng.random() < 0.3))


def sweep_cases(seed=SWEEP_SEED):
    rng = np.random.default_rng(seed)
    tag = "" if seed == SWEEP_SEED else "abcdefgh"[(seed - SWEEP_SEED) % 8]
    cases, i = [], 0
    while len(cases) < N_CASES:
        wl = _draw(rng, i, tag)
        i += 1
        if accepted(wl):
            cases.append(wl)
    return cases
