"""Seeded synthetic workloads for the conv1d -> GroupNorm path.

This module only describes shapes and draws random tensors.  It holds none of
the method's arithmetic (no convolution, statistic or normalisation), so both
the HIP path's callers and the oracle's callers may use it.

The shapes are those of the traces' problems (the POPCORNBENCH pages
"Kimi-K2.6 l2_p35" Conv1d->GroupNorm, "Kimi-K2.6 l1_p5" causal Conv1d and
"Kimi-K2.6 l2_p75" Linear->GroupNorm->min->+bias), plus a bf16 dilated
convolution with GroupNorm or LayerNorm over channels.  The benchmark's own
problem files are not used; these seeded tensors stand in for them.

Sampling recipe (all on the CPU, one ``torch.Generator`` seeded with ``seed``):
tensors are drawn in the order x, w, bias, gamma, beta, bias2, skipping the
ones a workload does not have.  U(+-b) is uniform on [-b, b]; N(0, s) has
standard deviation s.  x ~ N(0,1); w ~ U(+-1/sqrt(C_in*K)) unless the workload
fixes another bound; bias ~ U(+-0.1); gamma ~ U(0.5, 1.5); beta ~ N(0, 0.1);
bias2 ~ N(0,1).  For bf16 workloads x and w are drawn in fp32 and rounded to
bf16 (round to nearest even); parameters stay fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    C_in: int
    C_out: int
    T: int
    K: int
    stride: int = 1
    dilation: int = 1
    pad_left: int = 0
    pad_right: int = 0
    dtype: str = "f32"            # element type of x and w: "f32" or "bf16"
    out_dtype: str = "f32"        # element type of the output: "f32" or "bf16"
    norm: Optional[str] = "group"  # "group", "layer_channels" or None
    G: int = 1
    eps: float = 1e-5
    bias: bool = True             # conv bias present
    affine: bool = True           # gamma/beta present
    rowmin_bias: bool = False     # per-row min over channels + bias2 broadcast
    persistent: bool = True       # allow the persistent conv + normalisation route
    one_launch: bool = False      # Linear + GroupNorm + row-min as one launch
    cooperative: bool = False     # kernels whose workgroups wait on each other launched
                                  # through the runtime's cooperative launch
    channels_last: bool = False   # hand x to the library as [N, T, C_in]
    w_bound: Optional[float] = None

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Named workloads.  The names say what each one is and its sizes.
WORKLOADS = {
    w.name: w for w in [
        Workload("conv1d_gn_f32_n2_c16x32_t256_k3", N=2, C_in=16, C_out=32, T=256, K=3,
                 pad_left=1, pad_right=1, G=8),
        Workload("conv1d_gn_f32_n16_c128x256_t1024_k3", N=16, C_in=128, C_out=256, T=1024,
                 K=3, pad_left=1, pad_right=1, G=32),
        Workload("causal_conv1d_f32_n32_c256x256_t8192_k4", N=32, C_in=256, C_out=256,
                 T=8192, K=4, pad_left=3, pad_right=0, norm=None, G=1, bias=False,
                 affine=False, w_bound=1.0 / 32.0),
        Workload("gemm_gn_rowmin_bf16_m1024_n8192_k8192", N=1024, C_in=8192, C_out=8192,
                 T=1, K=1, dtype="bf16", G=512, bias=False, rowmin_bias=True),
        Workload("conv1d_gn_bf16_n64_c512x1024_t4096_k5d2", N=64, C_in=512, C_out=1024,
                 T=4096, K=5, dilation=2, pad_left=2, pad_right=2, dtype="bf16", G=32),
        Workload("conv1d_lnc_bf16_n64_c512x1024_t4096_k5d2", N=64, C_in=512, C_out=1024,
                 T=4096, K=5, dilation=2, pad_left=2, pad_right=2, dtype="bf16",
                 norm="layer_channels"),
        # beyond the pages' problems, at full scale: stride 2, 3 and 4, eight taps
        # at dilation 2 and at stride 4, seven causal taps, groups of 256 channels (spanning two
        # 128-channel tiles) and of 48 (not tiling them), channels-last input, fp32
        # with stride 2
        Workload("conv1d_gn_bf16_n32_c512x1024_t8192_k5s2", N=32, C_in=512, C_out=1024,
                 T=8192, K=5, stride=2, pad_left=2, pad_right=2, dtype="bf16", G=32),
        Workload("conv1d_gn_bf16_n32_c512x1024_t16384_k8s4", N=32, C_in=512, C_out=1024,
                 T=16384, K=8, stride=4, pad_left=2, pad_right=2, dtype="bf16", G=32),
        Workload("conv1d_gn_bf16_n32_c256x512_t4096_k8d2", N=32, C_in=256, C_out=512,
                 T=4096, K=8, dilation=2, pad_left=7, pad_right=7, dtype="bf16", G=16),
        Workload("conv1d_lnc_bf16_n32_c512x512_t4096_k7", N=32, C_in=512, C_out=512, T=4096,
                 K=7, pad_left=6, dtype="bf16", norm="layer_channels"),
        Workload("conv1d_gn_bf16_n32_c512x1024_t4096_k5d2_g4", N=32, C_in=512, C_out=1024,
                 T=4096, K=5, dilation=2, pad_left=4, pad_right=4, dtype="bf16", G=4),
        Workload("conv1d_gn_bf16_n16_c256x1536_t4096_k3_g32", N=16, C_in=256, C_out=1536,
                 T=4096, K=3, pad_left=1, pad_right=1, dtype="bf16", G=32),
        Workload("conv1d_lnc_bf16_nlc_n30_c384x768_t6000_k4s3", N=30, C_in=384, C_out=768,
                 T=6000, K=4, stride=3, pad_left=3, dtype="bf16", norm="layer_channels",
                 channels_last=True),
        Workload("conv1d_gn_f32_n16_c256x256_t8192_k4s2", N=16, C_in=256, C_out=256,
                 T=8192, K=4, stride=2, pad_left=3, G=32),
    ]
}

# The full-scale cases beyond the pages' problems (parity-tested on sampled
# outputs, timed by bench.py --mode generality).
GENERALITY = ("conv1d_gn_bf16_n32_c512x1024_t8192_k5s2",
              "conv1d_gn_bf16_n32_c512x1024_t16384_k8s4",
              "conv1d_gn_bf16_n32_c256x512_t4096_k8d2",
              "conv1d_lnc_bf16_n32_c512x512_t4096_k7",
              "conv1d_gn_bf16_n32_c512x1024_t4096_k5d2_g4",
              "conv1d_gn_bf16_n16_c256x1536_t4096_k3_g32",
              "conv1d_lnc_bf16_nlc_n30_c384x768_t6000_k4s3",
              "conv1d_gn_f32_n16_c256x256_t8192_k4s2")

# The headline workload timed by bench.py.
HEADLINE = "conv1d_gn_f32_n16_c128x256_t1024_k3"
# The small workload the oracle finishes in well under a second.
SMALL = "conv1d_gn_f32_n2_c16x32_t256_k3"


def _uniform(g, shape, lo, hi):
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    """Draw the workload's tensors on the CPU.

    Returns a dict with ``x`` and ``w`` in the workload's element type
    (float32 or bfloat16) and ``bias``, ``gamma``, ``beta``, ``bias2`` as
    float32 tensors or None."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((wl.N, wl.C_in, wl.T), generator=g, dtype=torch.float32)
    wb = wl.w_bound if wl.w_bound is not None else 1.0 / math.sqrt(wl.C_in * wl.K)
    w = _uniform(g, (wl.C_out, wl.C_in, wl.K), -wb, wb)
    out = {"x": x, "w": w, "bias": None, "gamma": None, "beta": None, "bias2": None}
    if wl.bias:
        out["bias"] = _uniform(g, (wl.C_out,), -0.1, 0.1)
    if wl.norm is not None and wl.affine:
        out["gamma"] = _uniform(g, (wl.C_out,), 0.5, 1.5)
        out["beta"] = torch.randn((wl.C_out,), generator=g, dtype=torch.float32) * 0.1
    if wl.rowmin_bias:
        out["bias2"] = torch.randn((wl.C_out,), generator=g, dtype=torch.float32)
    if wl.dtype == "bf16":
        out["x"] = out["x"].to(torch.bfloat16)
        out["w"] = out["w"].to(torch.bfloat16)
    elif wl.dtype != "f32":
        raise ValueError("unknown dtype %r" % (wl.dtype,))
    return out


def to_f64_numpy(t):
    """Exact widening of a CPU tensor (fp32 or bf16) to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
