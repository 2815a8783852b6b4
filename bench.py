#!/usr/bin/env python3
"""Benchmark of the conv1d -> GroupNorm path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one conv1d_gn_forward call (every kernel of the path) over one
batch of seeded synthetic input already resident in HBM.  W untimed steps,
then K timed steps.  Before each timed step the L2 caches and the Infinity
Cache are flushed (a 1 GiB buffer is read, so they hold only clean, unrelated
lines), and timed with HIP events on the launch stream as the time of
[flush, step] minus that of [flush] alone in the same rep: ``ms_per_step``
and ``value`` are the median over the K steps (the minimum is reported beside
it).  The same K steps back to back, caches warm, are
reported under ``warm``.  ``roofline`` places the dominant kernel against the
MI355X peak for both (``frac`` flushed, ``frac_warm``).

Without --workload the line is for the headline workload (fp32 conv1d +
GroupNorm, N16 C128->256 T1024 K3) and also carries
  - ``configs``: the same protocol on the causal conv, the Linear + GroupNorm
    + row-min, and the bf16 dilated conv with GroupNorm and with LayerNorm
    over channels;
  - ``passes``: the HBM-bound standalone passes (gn_stats, gn_apply,
    gn_apply_bf16) on tensors of the dilated-conv output's and the headline
    output's shapes, in GB/s of algorithmic bytes against the 8 TB/s peak;
  - ``cpu_baseline``: the fp64 oracle timed on this host's cores.

Other modes (used by the profiling runs recorded under profiles/):
    --mode copy     a plain device-to-device copy of known size, to scale the
                    FETCH_SIZE / WRITE_SIZE counters to bytes
    --mode passes   only the standalone HBM-bound passes
    --mode generality
                    the full-scale cases beyond the pages' problems (stride 2
                    and 3, eight taps at dilation 2, wide and non-tiling
                    groups, channels-last input, fp32 with stride 2)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused conv1d+GroupNorm TFLOP/s and GB/s at 1 GPU; % of MFMA/HBM roofline"
PEAKS = {  # MI355X published dense peaks
    "f32": ("mfma", 157.3, "TFLOP/s"),
    "bf16": ("mfma", 2500.0, "TFLOP/s"),
    "hbm": ("hbm", 8000.0, "GB/s"),
}
# kernel source files whose change invalidates stored counter readings
KERNEL_SOURCES = {
    "fused_single_pass": ["conv1d_implicit_gemm_amd/csrc/k_fused_gn.hip",
                          "conv1d_implicit_gemm_amd/csrc/common.hpp"],
}
# the workloads timed beside the headline, in the order of the pages' configurations
# (a ":out_bf16" suffix: the same workload with its output rounded to bf16)
EXTRA_CONFIGS = ["causal_conv1d_f32_n32_c256x256_t8192_k4",
                 "gemm_gn_rowmin_bf16_m1024_n8192_k8192",
                 "conv1d_gn_bf16_n64_c512x1024_t4096_k5d2",
                 "conv1d_lnc_bf16_n64_c512x1024_t4096_k5d2",
                 "conv1d_gn_bf16_n64_c512x1024_t4096_k5d2:out_bf16"]
FLUSH_BYTES = 1 << 30


def source_hash(route):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(route, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, route):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/<workload>.md), or None when absent or when the
    kernel's source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", workload + ".md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"```json counters\n(.*?)\n```", txt, flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if not KERNEL_SOURCES.get(route) or rec.get("kernel_source_sha256_16") != source_hash(route):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, flops, budget_s=10.0):
    """The oracle, as it stands, on the full workload, repeated until about
    budget_s seconds of wall time have passed (at least once), on all host
    threads; then once on one thread over the first sample only (the work per
    sample is the same for every sample), scaled to the same unit."""
    import oracle
    from conv1d_implicit_gemm_amd.workloads import to_f64_numpy as f
    args = dict(stride=wl.stride, dilation=wl.dilation, pad_left=wl.pad_left,
                pad_right=wl.pad_right, norm=wl.norm, G=wl.G, eps=wl.eps,
                gamma=f(inp["gamma"]), beta=f(inp["beta"]), bias2=f(inp["bias2"]))
    x, w, b = f(inp["x"]), f(inp["w"]), f(inp["bias"])
    threads = oracle.num_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(x, w, b, **args)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.forward(x[:1].copy(), w, b, **args)
        el1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "full workload (all %d samples), %d run(s) in %.1f s, fp64" % (wl.N, reps, el),
            "cpu_model": cpu_model(),
            "single_thread": {"value": flops / wl.N / el1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": "sample 0 of %d, one run in %.2f s, fp64" % (wl.N, el1)}}


class Timer:
    """Per-step timing on one stream with HIP events, caches flushed or warm."""

    def __init__(self, stream):
        import torch
        self.torch = torch
        self.stream = stream
        # filled once: reading it later leaves only clean, unrelated lines in
        # every cache level (no write-back of the flush lands in a timed step)
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda:0")

    def flush(self):
        self.torch.sum(self.buf, dim=0, out=self.sink)

    def flushed(self, op, reps, all_reps=False):
        """Median and minimum (ms) over reps steps, each run right after a
        flush.  An event between the flush and the step would add the step's
        launch latency to its time (the queue processes the event marker
        first), so each rep times [flush, step] and, just before it, [flush]
        alone, both after an untimed flush (so neither flush writes back what
        the step left dirty), and takes the difference.  The two flushes of a
        rep differ by a few microseconds, so a single rep's figure carries
        that much noise (all_reps: return the sorted per-rep figures too)."""
        torch = self.torch
        E = lambda: torch.cuda.Event(enable_timing=True)
        evs = [(E(), E(), E(), E()) for _ in range(reps)]
        torch.cuda.synchronize()
        for c, d, a, b in evs:
            self.flush()
            c.record(self.stream)
            self.flush()
            d.record(self.stream)
            a.record(self.stream)
            self.flush()
            op()
            b.record(self.stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) - c.elapsed_time(d) for c, d, a, b in evs)
        if all_reps:
            return statistics.median(t), t[0], t
        return statistics.median(t), t[0]

    def warm(self, op, reps):
        """Mean ms per step over reps back-to-back steps."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(self.stream)
        for _ in range(reps):
            op()
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps


def prepared(wl, persistent=True, one_launch=False):
    """The workload's seeded inputs on the device and a pre-marshalled call."""
    import torch
    import conv1d_implicit_gemm_amd as c1g
    from conv1d_implicit_gemm_amd.workloads import make_inputs
    inp = make_inputs(wl, 0)
    d = {k: (v.to("cuda:0").contiguous() if v is not None else None) for k, v in inp.items()}
    if wl.channels_last:  # the same values, laid out [N, T, C_in]
        d["x"] = d["x"].transpose(1, 2).contiguous()
    op = c1g.PreparedConv1dGN(d["x"], d["w"], d["bias"], stride=wl.stride,
                              dilation=wl.dilation, pad_left=wl.pad_left,
                              pad_right=wl.pad_right, norm=wl.norm, groups=wl.G, eps=wl.eps,
                              gamma=d["gamma"], beta=d["beta"], rowmin_bias=d["bias2"],
                              out_dtype=torch.bfloat16 if wl.out_dtype == "bf16"
                              else torch.float32, persistent=persistent,
                              one_launch=one_launch, channels_last=wl.channels_last)
    return inp, op


def measure(wl, op, timer, steps, warmup):
    """Flushed median/min and warm mean of one workload's step, with its roofline."""
    flops = 2 * wl.N * op.T_out * wl.C_out * wl.C_in * wl.K
    for _ in range(warmup):
        op()
    med, mn = timer.flushed(op, steps)
    warm = timer.warm(op, steps)
    bound, peak, unit = PEAKS[wl.dtype]
    algo_bytes = (wl.N * wl.C_in * wl.T * wl.elem_bytes + wl.C_out * wl.C_in * wl.K *
                  wl.elem_bytes + wl.N * wl.C_out * op.T_out * (2 if wl.out_dtype == "bf16" else 4))
    tf = lambda ms: flops / (ms * 1e-3) / 1e12
    return {"flops": flops, "ms_median": med, "ms_min": mn, "ms_warm": warm,
            "tflops": tf(med), "tflops_warm": tf(warm), "bound": bound, "peak": peak,
            "unit": unit, "frac": tf(med) / peak, "frac_warm": tf(warm) / peak,
            "algo_bytes": algo_bytes}


def config_entry(wl, op, m):
    """One workload's figures as they appear under ``configs`` and ``generality``."""
    return {"route": op.route, "dtype": wl.dtype, "out_dtype": wl.out_dtype,
            "ms_median": round(m["ms_median"], 5), "ms_min": round(m["ms_min"], 5),
            "ms_warm": round(m["ms_warm"], 5), "tflops": round(m["tflops"], 2),
            "tflops_warm": round(m["tflops_warm"], 2), "peak": m["peak"],
            "frac": round(m["frac"], 4), "frac_warm": round(m["frac_warm"], 4),
            "algorithmic_flops": m["flops"]}


def generality(timer, steps, warmup):
    """The full-scale cases beyond the pages' problems (stride 2, 3 and 4,
    eight taps at dilation 2 and at stride 4, groups spanning or not tiling the channel tiles,
    channels-last input, fp32 with stride 2), each step timed like the
    configurations, against its input type's MFMA peak."""
    import torch
    from conv1d_implicit_gemm_amd.workloads import GENERALITY, WORKLOADS
    res = {}
    for name in GENERALITY:
        wl = WORKLOADS[name]
        _, op = prepared(wl)
        res[name] = config_entry(wl, op, measure(wl, op, timer, steps, warmup))
        res[name]["shape"] = {k: getattr(wl, k) for k in (
            "N", "C_in", "C_out", "T", "K", "stride", "dilation", "pad_left", "pad_right",
            "norm", "G", "channels_last")}
        res[name]["shape"]["T_out"] = op.T_out
        del op
        torch.cuda.empty_cache()
    return res


def config_of(wl, op):
    return {"workload": wl.name, "N": wl.N, "C_in": wl.C_in, "C_out": wl.C_out, "T": wl.T,
            "T_out": op.T_out, "K": wl.K, "stride": wl.stride, "dilation": wl.dilation,
            "pad_left": wl.pad_left, "pad_right": wl.pad_right, "norm": wl.norm, "G": wl.G,
            "rowmin_bias": wl.rowmin_bias, "out_dtype": wl.out_dtype, "route": op.route,
            "parallelism": "single GPU"}


def passes(timer, steps, warmup):
    """The standalone HBM-bound passes on the dilated-conv output's shape
    ([64, 1024, 4092], G 32) and the headline output's ([16, 256, 1024], G 32):
    algorithmic bytes = every element read once (and written once by apply).
    Flushed figures: median and 10th / 90th percentiles over 5 x steps reps
    (a pass on the headline's shape takes ~5 us, the same order as the
    rep-to-rep noise of the flushed protocol, so one rep's figure, and the
    minimum, mean little there)."""
    import torch
    import conv1d_implicit_gemm_amd as c1g
    res = {}
    g = torch.Generator(device="cuda:0").manual_seed(0)
    for tag, (N, C, L, G) in (("dilated_conv_out", (64, 1024, 4092, 32)),
                              ("headline_out", (16, 256, 1024, 32))):
        y = torch.randn((N, C, L), generator=g, device="cuda:0")
        gam = torch.rand((C,), generator=g, device="cuda:0") + 0.5
        bet = torch.randn((C,), generator=g, device="cuda:0") * 0.1
        mean, rstd = c1g.gn_stats(y, G)
        out = torch.empty_like(y)
        yb = y.to(torch.bfloat16)
        outb = torch.empty_like(yb)
        n = N * C * L
        # direct C-ABI calls with pre-marshalled arguments: per-call host work
        # stays far below the kernels' time
        lib = c1g.load_library()
        ws_bytes = lib.c1g_gn_stats_workspace_size(N, C, L, G)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda:0")
        st_mean, st_rstd = torch.empty_like(mean), torch.empty_like(rstd)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        sp = ctypes.c_void_p(timer.stream.cuda_stream)
        a_stats = (N, C, L, G, 1e-5, P(y), P(st_mean), P(st_rstd), P(ws), ws_bytes, sp)
        a_apply = (N, C, L, G, P(y), P(mean), P(rstd), P(gam), P(bet), P(out), sp)
        a_applyb = (N, C, L, G, P(yb), P(mean), P(rstd), P(gam), P(bet), P(outb), sp)

        def call(fn, a):
            def run():
                if fn(*a) != 0:
                    raise RuntimeError("%s failed" % fn.__name__)
            return run
        cases = [("gn_stats", call(lib.gn_stats, a_stats), 4 * n),
                 ("gn_apply", call(lib.gn_apply, a_apply), 8 * n),
                 ("gn_apply_bf16", call(lib.gn_apply_bf16, a_applyb), 4 * n)]
        for name, fn, nbytes in cases:
            for _ in range(warmup):
                fn()
            med, _, t = timer.flushed(fn, 5 * steps, all_reps=True)
            warm = timer.warm(fn, steps)
            gbps = nbytes / (med * 1e-3) / 1e9
            p10, p90 = t[len(t) // 10], t[(9 * len(t)) // 10]
            res["%s_%s" % (name, tag)] = {
                "shape": [N, C, L], "G": G, "algorithmic_bytes": nbytes,
                "ms_median": round(med, 5), "ms_p10": round(p10, 5), "ms_p90": round(p90, 5),
                "ms_warm": round(warm, 5),
                "gbps": round(gbps, 1), "peak_gbps": PEAKS["hbm"][1],
                "frac": round(gbps / PEAKS["hbm"][1], 4)}
        torch.cuda.synchronize()
        del y, out, yb, outb, ws
    return res


def copy_mode(args):
    import torch
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, device="cuda:0", dtype=torch.float32).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": args.steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="time this workload alone (no configs, passes or CPU baseline)")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy", "passes", "generality"])
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"],
                    help="element type of the output (bf16: rounded to nearest even)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-persistent", action="store_true",
                    help="bf16 conv + GroupNorm/LayerNorm: time the multi-kernel split route "
                         "instead of the persistent single-kernel one")
    ap.add_argument("--one-launch", action="store_true",
                    help="Linear + GroupNorm + row-min: one launch instead of the GEMM and a "
                         "broadcast kernel")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        return copy_mode(args)
    steps = max(args.steps, 1)

    import torch
    from conv1d_implicit_gemm_amd.workloads import HEADLINE, WORKLOADS

    stream = torch.cuda.current_stream("cuda:0")
    timer = Timer(stream)
    if args.mode == "passes":
        print(json.dumps({"mode": "passes", "steps": steps,
                          "passes": passes(timer, steps, args.warmup)}), flush=True)
        return
    if args.mode == "generality":
        print(json.dumps({"mode": "generality", "steps": steps, "warmup": args.warmup,
                          "generality": generality(timer, steps, args.warmup)}), flush=True)
        return

    name = args.workload or HEADLINE
    wl = WORKLOADS[name].replace(out_dtype=args.out_dtype)
    inp, op = prepared(wl, persistent=not args.no_persistent, one_launch=args.one_launch)
    m = measure(wl, op, timer, steps, args.warmup)
    # stored counters were taken with an fp32 output
    traffic = stored_traffic(name, op.route) if wl.out_dtype == "f32" else None
    res = {
        "metric": METRIC, "value": round(m["tflops"], 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(m["ms_median"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded; shapes of the pages' workloads)",
        "config": config_of(wl, op),
        "timing": {"protocol": "each of the %d timed steps right after reading a 1 GiB "
                               "buffer (L2 and Infinity Cache then hold only clean unrelated "
                               "lines), HIP events on the launch stream: time of [flush, step] "
                               "minus time of [flush] in the same rep (no event between flush "
                               "and step, so its launch overlaps the flush as in a stream of "
                               "work); value and ms_per_step are the median" % steps,
                   "ms_min": round(m["ms_min"], 5),
                   "warm": {"ms_per_step": round(m["ms_warm"], 5),
                            "value": round(m["tflops_warm"], 3),
                            "note": "the same steps back to back, caches warm"}},
        "gbps_algorithmic": round(m["algo_bytes"] / (m["ms_median"] * 1e-3) / 1e9, 1),
        "roofline": {"bound": m["bound"], "achieved": round(m["tflops"], 3), "peak": m["peak"],
                     "unit": m["unit"], "frac": round(m["frac"], 4), "traffic": traffic,
                     "kernel_ms": round(m["ms_median"], 5),
                     "achieved_warm": round(m["tflops_warm"], 3),
                     "frac_warm": round(m["frac_warm"], 4),
                     "kernel_ms_warm": round(m["ms_warm"], 5),
                     "algorithmic_flops_per_launch": m["flops"],
                     "note": "one launch per step on this route: the step's event time is "
                             "the kernel's" if op.route == "fused_single_pass" else
                             "several launches per step: fractions are of the whole step"},
    }
    if args.workload is None:
        cfgs = {}
        for cname in EXTRA_CONFIGS:
            base, _, variant = cname.partition(":")
            cwl = WORKLOADS[base]
            if variant == "out_bf16":
                cwl = cwl.replace(out_dtype="bf16")
            _, cop = prepared(cwl)
            cfgs[cname] = config_entry(cwl, cop, measure(cwl, cop, timer, steps, args.warmup))
            del cop
            torch.cuda.empty_cache()
        res["configs"] = cfgs
        res["passes"] = passes(timer, steps, args.warmup)
    if not args.no_cpu_baseline and args.workload is None:
        res["cpu_baseline"] = cpu_baseline(wl, inp, m["flops"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
