"""HIP graph capture of the library's calls.  The entry points enqueue
kernels only (counters are cleared by fill kernels, never by memset nodes),
so a prepared call can be captured once and replayed.  Each case captures a
PreparedConv1dGN call (and one allocation-free call) on a side stream, then
replays the graph several times with the program's own eager work and
synchronisations in between, the output poisoned with NaN before every
replay; every replay must equal the eager result bit for bit.  Also: calls
from several host threads at once, each on its own stream (the routes whose
workgroups wait on each other with cooperative launches)."""
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g
from conv1d_implicit_gemm_amd.workloads import Workload, make_inputs
from tests.gpu_util import DEV, announce, to_dev

pytestmark = pytest.mark.gpu

BF = dict(dtype="bf16")
# (workload, the route it takes)
CASES = [
    (Workload("graph_fused_fp32", N=2, C_in=32, C_out=64, T=300, K=3, pad_left=1,
              pad_right=1, G=8), "fused_single_pass"),
    (Workload("graph_split_fp32_rowmin", N=2, C_in=24, C_out=48, T=200, K=4, pad_left=3, G=6,
              rowmin_bias=True), "split"),
    (Workload("graph_split_bf16_gn", N=3, C_in=72, C_out=160, T=1300, K=5, dilation=2,
              pad_left=2, pad_right=2, G=8, persistent=False, **BF), "split"),
    (Workload("graph_persistent_bf16_gn", N=3, C_in=72, C_out=256, T=1300, K=5, dilation=2,
              pad_left=2, pad_right=2, G=16, **BF), "fused_persistent"),
    (Workload("graph_persistent_bf16_ln", N=2, C_in=40, C_out=272, T=700, K=5, dilation=2,
              pad_left=2, pad_right=2, norm="layer_channels", **BF), "fused_persistent"),
    (Workload("graph_gemm_rowmin", N=300, C_in=256, C_out=512, T=1, K=1, G=32,
              rowmin_bias=True, **BF), "gemm_rows"),
    (Workload("graph_gemm_rowmin_one_launch", N=300, C_in=256, C_out=512, T=1, K=1, G=32,
              rowmin_bias=True, one_launch=True, **BF), "gemm_rows"),
]
REPLAYS = 3


def _tensors(wl, inp):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x, w = to_dev(inp["x"]).to(dt), to_dev(inp["w"]).to(dt)
    return (x, w) + tuple(to_dev(inp[k]) for k in ("bias", "gamma", "beta", "bias2"))


def _replay_and_compare(g, out, eager):
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()  # the program's own eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager call" % r
        del junk


@pytest.mark.parametrize("wl,route", CASES, ids=[c[0].name for c in CASES])
def test_graph_replays_match_eager(wl, route):
    announce("graph capture", wl.name)
    inp = make_inputs(wl, 11)
    x, w, b, ga, be, b2 = _tensors(wl, inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # the prepared call enqueues on the stream current here
        op = c1g.PreparedConv1dGN(x, w, b, stride=wl.stride, dilation=wl.dilation,
                                  pad_left=wl.pad_left, pad_right=wl.pad_right, norm=wl.norm,
                                  groups=wl.G, eps=wl.eps, gamma=ga, beta=be, rowmin_bias=b2,
                                  persistent=wl.persistent, one_launch=wl.one_launch)
        assert op.route == route
        for _ in range(2):
            op()
    s.synchronize()
    eager = op.out.clone()
    assert torch.isfinite(eager).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        op()
    _replay_and_compare(g, op.out, eager)


def test_graph_replays_noalloc():
    """The allocation-free entry point, made for callers such as graph
    capture: its first call (outside the capture) looks up the device
    scratch; captured calls then allocate nothing."""
    wl = CASES[3][0]  # the persistent route: pack kernels, then the waiting conv
    announce("graph capture, allocation-free entry point", wl.name)
    inp = make_inputs(wl, 12)
    x, w, b, ga, be, _ = _tensors(wl, inp)
    kw = dict(dilation=wl.dilation, pad_left=wl.pad_left, pad_right=wl.pad_right,
              norm=wl.norm, groups=wl.G, eps=wl.eps, gamma=ga, beta=be)
    T_out = c1g.out_len(c1g.make_desc(wl.N, wl.C_in, wl.C_out, wl.T, wl.K,
                                      dilation=wl.dilation, pad_left=wl.pad_left,
                                      pad_right=wl.pad_right))
    out = torch.empty((wl.N, wl.C_out, T_out), device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            c1g.conv1d_gn_forward_noalloc(x, w, b, out=out, **kw)
    s.synchronize()
    eager = out.clone()
    ref = c1g.conv1d_gn_forward(x, w, b, **kw)
    torch.cuda.synchronize()
    assert torch.equal(eager, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c1g.conv1d_gn_forward_noalloc(x, w, b, out=out, **kw)
    _replay_and_compare(g, out, eager)


def test_concurrent_host_threads():
    """Entry points called concurrently from several host threads, each on its
    own stream with its own tensors (routes without waits between
    workgroups), give the same bits as the same calls made one at a time."""
    import threading
    cases = [c for c, r in CASES if r in ("fused_single_pass", "split", "gemm_rows")
             and not c.one_launch]
    announce("concurrent host threads", len(cases), "cases")
    jobs = []
    for i, wl in enumerate(cases * 2):
        inp = make_inputs(wl, 20 + i)
        x, w, b, ga, be, b2 = _tensors(wl, inp)
        kw = dict(stride=wl.stride, dilation=wl.dilation, pad_left=wl.pad_left,
                  pad_right=wl.pad_right, norm=wl.norm, groups=wl.G, eps=wl.eps, gamma=ga,
                  beta=be, rowmin_bias=b2, persistent=False)
        ref = c1g.conv1d_gn_forward(x, w, b, **kw)
        jobs.append((x, w, b, kw, ref))
    torch.cuda.synchronize()
    results = [None] * len(jobs)
    errors = []

    def run(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [c1g.conv1d_gn_forward(x, w, b, **kw) for x, w, b, kw, _ in [jobs[k]] * 3]
            s.synchronize()
            results[k] = outs
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (_, _, _, _, ref), outs in zip(jobs, results):
        for o in outs:
            assert torch.equal(o, ref)


def test_concurrent_cooperative_launches():
    """The routes whose workgroups wait on each other, called concurrently
    from several host threads with cooperative=True (what callers that share
    the device with other work are told to set): the runtime keeps each
    launch's workgroups co-resident, so every call gives the bits of the same
    call made alone (a wait that gave up would have written NaN)."""
    import threading
    cases = [c for c, r in CASES if r == "fused_persistent" or c.one_launch]
    announce("concurrent cooperative launches", len(cases), "cases")
    jobs = []
    for i, wl in enumerate(cases * 2):
        inp = make_inputs(wl, 40 + i)
        x, w, b, ga, be, b2 = _tensors(wl, inp)
        kw = dict(stride=wl.stride, dilation=wl.dilation, pad_left=wl.pad_left,
                  pad_right=wl.pad_right, norm=wl.norm, groups=wl.G, eps=wl.eps, gamma=ga,
                  beta=be, rowmin_bias=b2, one_launch=wl.one_launch, cooperative=True)
        ref = c1g.conv1d_gn_forward(x, w, b, **kw)
        jobs.append((x, w, b, kw, ref))
    torch.cuda.synchronize()
    assert all(torch.isfinite(j[4]).all() for j in jobs)
    results = [None] * len(jobs)
    errors = []

    def run(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [c1g.conv1d_gn_forward(x, w, b, **kw) for x, w, b, kw, _ in [jobs[k]] * 3]
            s.synchronize()
            results[k] = outs
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (_, _, _, _, ref), outs in zip(jobs, results):
        for o in outs:
            assert torch.equal(o, ref)
