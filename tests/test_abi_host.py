"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and its host-only planning and validation behave as documented.
No compute call is made (there is no GPU here)."""
import ctypes
import os
import re

import pytest

import conv1d_implicit_gemm_amd as c1g
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv1d_gn.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_0-9]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_lists_every_binding_export():
    assert header_functions() == sorted(c1g.EXPORTS)


@pytest.mark.parametrize("name", header_functions())
def test_library_exports_symbol(name):
    lib = c1g.load_library()
    assert hasattr(lib, name), name
    assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings():
    lib = c1g.load_library()
    for code, text in c1g.STATUS.items():
        assert lib.c1g_status_string(code).decode() == text


@pytest.mark.parametrize("T,K,s,d,pl,pr", [
    (1024, 3, 1, 1, 1, 1), (8192, 4, 1, 1, 3, 0), (1, 1, 1, 1, 0, 0), (4096, 5, 1, 2, 2, 2),
    (7, 3, 2, 1, 0, 0), (10, 4, 3, 2, 1, 2), (5, 3, 1, 3, 0, 0), (2, 5, 1, 1, 0, 0)])
def test_out_len_matches_oracle(T, K, s, d, pl, pr):
    desc = c1g.ConvDesc(2, 3, 4, T, K, s, d, pl, pr, c1g.C1G_F32)
    assert c1g.out_len(desc) == oracle.out_len(T, K, s, d, pl, pr)


def _desc(**kw):
    base = dict(N=2, C_in=16, C_out=32, T=256, K=3, stride=1, dilation=1, pad_left=1,
                pad_right=1, dtype=c1g.C1G_F32, out_dtype=c1g.C1G_F32, x_layout=0)
    base.update(kw)
    return c1g.ConvDesc(base["N"], base["C_in"], base["C_out"], base["T"], base["K"],
                        base["stride"], base["dilation"], base["pad_left"], base["pad_right"],
                        base["dtype"], base["out_dtype"], base["x_layout"])


@pytest.mark.parametrize("kw", [dict(N=-1), dict(C_in=0), dict(C_out=0), dict(T=0), dict(K=0),
                                dict(stride=0), dict(dilation=0), dict(pad_left=-1),
                                dict(pad_right=-1), dict(T=2, K=5, pad_left=0, pad_right=0)])
def test_invalid_geometry(kw):
    d = _desc(**kw)
    assert c1g.check(d) == 1
    assert c1g.route(d) == "invalid"
    assert c1g.out_len(d) == -1


def test_empty_batch_is_a_no_op():
    """N = 0: valid on every route's geometry, route "empty", no workspace,
    and the other arguments are still checked; the standalone passes return
    OK without touching their (NULL) pointers."""
    lin = dict(C_in=256, C_out=512, T=1, K=1, pad_left=0, pad_right=0, dtype=c1g.C1G_BF16)
    cases = [(_desc(N=0), c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)),
             (_desc(N=0, C_in=512, C_out=1024, T=4096, K=5, dilation=2, pad_left=4,
                    pad_right=4, dtype=c1g.C1G_BF16), c1g.NormDesc(c1g.NORM_LAYER_CHANNELS, 0, 1e-5, 0)),
             (_desc(N=0, **lin), c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 1)),
             (_desc(N=0), None)]
    for d, nd in cases:
        assert c1g.out_len(d) == c1g.out_len(_desc(**{k: getattr(d, k) for k in (
            "C_in", "C_out", "T", "K", "stride", "dilation", "pad_left", "pad_right")}))
        assert c1g.route(d, nd) == "empty"
        assert c1g.check(d, nd, 0) == 0
        assert c1g.conv1d_workspace_size(d) == 0
        if nd is not None:
            assert c1g.conv1d_gn_workspace_size(d, nd) == 0
    assert c1g.check(_desc(N=0), c1g.NormDesc(c1g.NORM_GROUP, 5, 1e-5, 0)) == 1  # 32 % 5
    assert c1g.check(_desc(N=0, dtype=7)) == 2
    lib = c1g.load_library()
    assert lib.c1g_gn_stats_workspace_size(0, 32, 100, 8) == 0
    assert lib.gn_stats(0, 32, 100, 8, 1e-5, None, None, None, None, 0, None) == 0
    assert lib.gn_stats(0, 32, 100, 8, 0.0, None, None, None, None, 0, None) == 1    # eps
    assert lib.gn_apply(0, 32, 100, 8, None, None, None, None, None, None, None) == 0
    assert lib.gn_apply(0, 32, 100, 5, None, None, None, None, None, None, None) == 1
    assert lib.gn_apply_bf16(0, 32, 100, 8, None, None, None, None, None, None, None) == 0
    for fn in (lib.conv1d_forward,):
        assert fn(ctypes.byref(_desc(N=0)), None, None, None, None, None, 0, None) == 0
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    assert lib.conv1d_gn_forward(ctypes.byref(_desc(N=0)), ctypes.byref(gn), None, None, None,
                                 None, None, None, None, None, None, None, 0, None) == 0
    assert lib.conv1d_gn_forward_noalloc(ctypes.byref(_desc(N=0)), ctypes.byref(gn), None, None,
                                         None, None, None, None, None, None, None, None) == 0


def test_invalid_norm_args():
    d = _desc()
    assert c1g.check(d, c1g.NormDesc(c1g.NORM_GROUP, 5, 1e-5, 0)) == 1   # 32 % 5
    assert c1g.check(d, c1g.NormDesc(c1g.NORM_GROUP, 0, 1e-5, 0)) == 1
    assert c1g.check(d, c1g.NormDesc(c1g.NORM_GROUP, 8, 0.0, 0)) == 1    # eps must be > 0
    assert c1g.check(d, c1g.NormDesc(c1g.NORM_GROUP, 8, float("nan"), 0)) == 1
    assert c1g.check(d, c1g.NormDesc(7, 8, 1e-5, 0)) == 1
    assert c1g.check(d, c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 9)) == 1
    assert c1g.check(_desc(dtype=7)) == 2
    assert c1g.check(_desc(out_dtype=7)) == 2
    assert c1g.check(_desc(out_dtype=c1g.C1G_BF16)) == 0


def test_routes():
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    assert c1g.route(_desc(), gn) == "fused_single_pass"
    big = _desc(N=16, C_in=128, C_out=256, T=1024)
    assert c1g.route(big, c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 0)) == "fused_single_pass"
    # C_out/G = 3 does not divide 16 -> split path
    assert c1g.route(_desc(C_out=24), gn) == "split"
    # too long for the on-chip slab -> split path
    assert c1g.route(_desc(T=1500), gn) == "split"
    assert c1g.route(_desc(), c1g.NormDesc(c1g.NORM_LAYER_CHANNELS, 0, 1e-5, 0)) == "split"
    assert c1g.route(_desc(), c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 1)) == "split"
    assert c1g.route(_desc()) == "conv_only"
    bf = c1g.C1G_BF16
    lin = _desc(N=1024, C_in=8192, C_out=8192, T=1, K=1, pad_left=0, pad_right=0, dtype=bf)
    assert c1g.route(lin, c1g.NormDesc(c1g.NORM_GROUP, 512, 1e-5, 1)) == "gemm_rows"
    assert c1g.route(lin) == "gemm_rows"
    conv = _desc(N=64, C_in=512, C_out=1024, T=4096, K=5, dilation=2, pad_left=2,
                 pad_right=2, dtype=bf)
    # bf16: the persistent conv normalises in registers (64 tiles per sample)
    assert c1g.route(conv, c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 0)) == "fused_persistent"
    assert c1g.route(conv, c1g.NormDesc(c1g.NORM_LAYER_CHANNELS, 0, 1e-5, 0)) == \
        "fused_persistent"
    no_p = c1g.FLAG_NO_PERSISTENT
    assert c1g.route(conv, c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 0, no_p)) == "split"
    assert c1g.route(conv, c1g.NormDesc(c1g.NORM_LAYER_CHANNELS, 0, 1e-5, 0, no_p)) == "split"
    # groups that straddle the 128-channel tiles (C_out/G = 48) stay
    # persistent; the row-min epilogue, or more than 256 tiles per sample: split
    assert c1g.route(_desc(C_in=64, C_out=192, T=512, dtype=bf),
                     c1g.NormDesc(c1g.NORM_GROUP, 4, 1e-5, 0)) == "fused_persistent"
    assert c1g.route(conv, c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 1)) == "split"
    assert c1g.route(_desc(C_in=64, C_out=1024, T=140000, dtype=bf),
                     c1g.NormDesc(c1g.NORM_LAYER_CHANNELS, 0, 1e-5, 0)) == "split"
    # groups spanning whole tiles (C_out/G = 256) stay persistent
    assert c1g.route(conv, c1g.NormDesc(c1g.NORM_GROUP, 4, 1e-5, 0)) == "fused_persistent"
    assert c1g.route(conv) == "conv_only"


def test_workspace_sizes():
    d = _desc(C_out=24)
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    need = c1g.conv1d_gn_workspace_size(d, gn)
    assert need > 0
    assert c1g.check(d, gn, need) == 0
    assert c1g.check(d, gn, need - 1) == 3
    # fused route needs none
    assert c1g.conv1d_gn_workspace_size(_desc(), gn) == 0
    assert c1g.conv1d_workspace_size(_desc()) > 0


def test_unsupported_sizes():
    # taps beyond the LDS weight image
    assert c1g.check(_desc(K=9, pad_left=4, pad_right=4)) == 2
    # input window wider than any tile variant
    assert c1g.check(_desc(stride=8, T=4096)) == 2
    # bf16 convolution: up to 8 taps (6..8 on 128-position tiles), not 9
    assert c1g.check(_desc(K=8, pad_left=3, pad_right=4, dtype=c1g.C1G_BF16)) == 0
    assert c1g.check(_desc(K=9, pad_left=4, pad_right=4, dtype=c1g.C1G_BF16)) == 2
    # bf16, 8 taps: the window of a 128-position tile, 127 + 7*dilation + 1
    # input rows, must fit 224 rows
    assert c1g.check(_desc(K=8, dilation=13, pad_left=0, pad_right=0, T=4096,
                           dtype=c1g.C1G_BF16)) == 0
    assert c1g.check(_desc(K=8, dilation=14, pad_left=0, pad_right=0, T=4096,
                           dtype=c1g.C1G_BF16)) == 2
    # bf16, 5 taps on a 512-position tile: 511 + 4*dilation + 1 <= 544 rows,
    # else the 128-position tile
    assert c1g.check(_desc(K=5, dilation=8, T=8192, dtype=c1g.C1G_BF16)) == 0
    assert c1g.check(_desc(K=5, dilation=9, T=8192, dtype=c1g.C1G_BF16)) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 2, 8)
    w = torch.zeros(3, 2, 3)
    with pytest.raises(ValueError):
        c1g.conv1d_forward(x, w)


def test_pointer_checks_fail_before_any_launch():
    """Validation rejects bad pointers without touching memory or the device:
    fake addresses are safe because nothing is dereferenced or launched."""
    lib = c1g.load_library()
    d = _desc()
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    P = ctypes.c_void_p
    good = P(0x10000)
    odd = P(0x10002)      # 2-byte aligned: not enough for fp32
    # missing required pointers
    assert lib.conv1d_forward(ctypes.byref(d), None, good, None, good, good, 1 << 30, None) == 1
    assert lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(gn), good, good, None, None, None,
                                 None, None, None, None, None, 0, None) == 1
    # misaligned fp32 tensors
    assert lib.conv1d_forward(ctypes.byref(d), odd, good, None, good, good, 1 << 30, None) == 4
    assert lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(gn), good, good, None, odd, None,
                                 None, good, None, None, None, 0, None) == 4
    # workspace too small
    need = c1g.conv1d_workspace_size(d)
    assert lib.conv1d_forward(ctypes.byref(d), good, good, None, good, good, need - 1, None) == 3
    assert lib.conv1d_forward(ctypes.byref(d), good, good, None, good, None, 0, None) == 3
    # row-min epilogue without bias2
    rm = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 1)
    assert lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(rm), good, good, None, None, None,
                                 None, good, None, None, good, 1 << 30, None) == 1
    # standalone GroupNorm entry points
    assert lib.gn_stats(2, 32, 10, 5, 1e-5, good, good, good, None, 0, None) == 1
    assert lib.gn_stats(2, 32, 10, 8, 1e-5, odd, good, good, None, 0, None) == 4
    # groups of more than 32768 values need the two-stage workspace
    need = lib.c1g_gn_stats_workspace_size(1, 64, 4096, 1)
    assert need == 256                       # 8 slices x 8 bytes, rounded up to 256
    assert lib.c1g_gn_stats_workspace_size(2, 32, 1000, 8) == 0
    assert lib.c1g_gn_stats_workspace_size(2, 32, 1000, 5) == 0   # invalid: 0
    assert lib.gn_stats(1, 64, 4096, 1, 1e-5, good, good, good, None, 0, None) == 3
    assert lib.gn_stats(1, 64, 4096, 1, 1e-5, good, good, good, good, need - 8, None) == 3
    assert lib.gn_stats(1, 64, 4096, 1, 1e-5, good, good, good, P(0x10010), need, None) == 4
    assert lib.gn_stats(1, 64, 4096, 1, 0.0, good, good, good, good, need, None) == 1
    assert lib.gn_apply(2, 32, 10, 8, good, good, good, None, None, None, None) == 1
    assert lib.gn_apply(2, 32, 10, 8, good, odd, good, None, None, good, None) == 4
    # bf16 outputs need 2-byte alignment only
    odd1 = P(0x10001)
    db = _desc(out_dtype=c1g.C1G_BF16)
    assert lib.conv1d_forward(ctypes.byref(db), good, good, None, odd1, good, 1 << 30, None) == 4
    assert lib.conv1d_gn_forward(ctypes.byref(db), ctypes.byref(gn), good, good, None, None,
                                 None, None, odd1, None, None, good, 1 << 30, None) == 4
    assert lib.gn_apply_bf16(2, 32, 10, 5, good, good, good, None, None, good, None) == 1
    assert lib.gn_apply_bf16(2, 32, 10, 8, None, good, good, None, None, good, None) == 1
    assert lib.gn_apply_bf16(2, 32, 10, 8, odd1, good, good, None, None, good, None) == 4
    assert lib.gn_apply_bf16(2, 32, 10, 8, good, odd, good, None, None, good, None) == 4


def test_bf16_output_workspace():
    """A bf16 out adds an fp32 y to the workspace only where an unfused
    epilogue follows the Linear-layer GEMM; elsewhere y lives in out."""
    lin = dict(N=64, C_in=256, C_out=512, T=1, K=1, pad_left=0, pad_right=0, dtype=c1g.C1G_BF16)
    f32, b16 = _desc(**lin), _desc(out_dtype=c1g.C1G_BF16, **lin)
    unfused = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)    # 64 channels per group
    fused = c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 1)     # 16 per group + row-min
    assert c1g.route(b16, unfused) == "gemm_rows"
    extra = c1g.conv1d_gn_workspace_size(b16, unfused) - c1g.conv1d_gn_workspace_size(f32, unfused)
    assert 64 * 512 * 4 <= extra < 64 * 512 * 4 + 256
    assert c1g.conv1d_gn_workspace_size(b16, fused) == c1g.conv1d_gn_workspace_size(f32, fused)
    assert c1g.conv1d_workspace_size(b16) == c1g.conv1d_workspace_size(f32) == 0
    conv = dict(N=2, C_in=64, C_out=128, T=300, K=5, dilation=2, pad_left=2, pad_right=2)
    for dt in (c1g.C1G_F32, c1g.C1G_BF16):
        a, b = _desc(dtype=dt, **conv), _desc(dtype=dt, out_dtype=c1g.C1G_BF16, **conv)
        for nd in (c1g.NormDesc(c1g.NORM_GROUP, 4, 1e-5, 0),     # 32 channels per group
                   c1g.NormDesc(c1g.NORM_GROUP, 4, 1e-5, 0, c1g.FLAG_NO_PERSISTENT),
                   c1g.NormDesc(c1g.NORM_LAYER_CHANNELS, 0, 1e-5, 1)):
            assert c1g.route(a, nd) == c1g.route(b, nd) != "gemm_rows"
            assert c1g.conv1d_gn_workspace_size(a, nd) == c1g.conv1d_gn_workspace_size(b, nd)


def test_conv_desc_abi_size():
    """c1g_conv_desc: four int64 fields then eight int32 fields, 64 bytes."""
    assert ctypes.sizeof(c1g.ConvDesc) == 64
    assert c1g.ConvDesc.x_layout.offset == 60


def test_channels_last_planning():
    """A channels-last x: an invalid layout code is an argument error; fp32
    routes add x transposed ([N, C_in, T] fp32, 256-byte aligned) to the front
    of the workspace, including the otherwise workspace-free fused route;
    bf16 routes build their input image from either layout at no extra size;
    with T = 1 the layouts are the same bytes and nothing changes."""
    assert c1g.check(_desc(x_layout=2)) == 1
    assert c1g.check(_desc(x_layout=-1)) == 1
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    cases = [dict(), dict(C_out=24), dict(N=3, C_in=40, C_out=64, T=513, K=4, pad_left=3,
                                           pad_right=0)]
    for kw in cases:
        a, b = _desc(**kw), _desc(x_layout=c1g.LAYOUT_NLC, **kw)
        xt = -(-(a.N * a.C_in * a.T * 4) // 256) * 256
        for nd in (gn, None):
            if nd is None:
                wa, wb = c1g.conv1d_workspace_size(a), c1g.conv1d_workspace_size(b)
            else:
                assert c1g.route(a, nd) == c1g.route(b, nd)
                wa, wb = c1g.conv1d_gn_workspace_size(a, nd), c1g.conv1d_gn_workspace_size(b, nd)
            assert wb == wa + xt, (kw, nd)
    for kw in (dict(dtype=c1g.C1G_BF16), dict(dtype=c1g.C1G_BF16, C_out=256, T=2000)):
        a, b = _desc(**kw), _desc(x_layout=c1g.LAYOUT_NLC, **kw)
        assert c1g.route(a, gn) == c1g.route(b, gn)
        assert c1g.conv1d_gn_workspace_size(a, gn) == c1g.conv1d_gn_workspace_size(b, gn)
        assert c1g.conv1d_workspace_size(a) == c1g.conv1d_workspace_size(b)
    lin = dict(N=64, C_in=256, C_out=512, T=1, K=1, pad_left=0, pad_right=0)
    for dt in (c1g.C1G_F32, c1g.C1G_BF16):
        a, b = _desc(dtype=dt, **lin), _desc(dtype=dt, x_layout=c1g.LAYOUT_NLC, **lin)
        assert c1g.route(a, gn) == c1g.route(b, gn)
        assert c1g.conv1d_gn_workspace_size(a, gn) == c1g.conv1d_gn_workspace_size(b, gn)


def test_noalloc_rejects_before_any_launch():
    """conv1d_gn_forward_noalloc checks its pointers and refuses problems whose
    workspace exceeds its static scratch before anything touches a device
    (fake addresses are safe: nothing is dereferenced or launched)."""
    lib = c1g.load_library()
    P = ctypes.c_void_p
    good, odd = P(0x10000), P(0x10002)
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    d = _desc(dtype=c1g.C1G_BF16)
    f = lib.conv1d_gn_forward_noalloc
    assert f(ctypes.byref(d), ctypes.byref(gn), None, good, None, None, None, None, good,
             None, None, None) == 1
    assert f(ctypes.byref(d), ctypes.byref(gn), good, good, None, None, None, None, odd,
             None, None, None) == 4
    # the dilated-conv workload needs ~290 MB of workspace: more than the scratch
    big = _desc(N=64, C_in=512, C_out=1024, T=4096, K=5, dilation=2, pad_left=2, pad_right=2,
                dtype=c1g.C1G_BF16)
    gn32 = c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 0)
    assert c1g.conv1d_gn_workspace_size(big, gn32) > c1g.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), ctypes.byref(gn32), good, good, None, None, None, None, good,
             None, None, None) == 3
    # invalid geometry is reported as such
    bad = _desc(T=2, K=5, pad_left=0, pad_right=0)
    assert f(ctypes.byref(bad), ctypes.byref(gn), good, good, None, None, None, None, good,
             None, None, None) == 1


def test_oversized_arguments_are_refused_not_wrapped():
    """Sizes whose products would wrap 64 bits are refused (C1G_ERR_UNSUPPORTED,
    workspace size 0, c1g_out_len -1 for a length past 2^62), never accepted
    as the small sizes they wrap to.  Validation fails before any pointer is
    read or anything is launched, so fake aligned addresses are safe."""
    assert c1g.out_len(_desc(T=2 ** 63 - 1)) == -1
    assert c1g.out_len(_desc(T=2 ** 62, K=1, pad_left=0, pad_right=0)) == 2 ** 62
    for kw in (dict(T=2 ** 41, K=1, pad_left=0, pad_right=0, stride=2 ** 20, N=1, C_out=1),
               # x of 2^59 elements (2^30 outputs)
               dict(N=1, C_in=2 ** 29, C_out=1, T=2 ** 30, K=1, pad_left=0, pad_right=0),
               # a channels-last fp32 x whose transpose would take 2^88 bytes
               dict(N=65535, C_in=2 ** 30, C_out=1, T=2 ** 40, K=1, pad_left=0, pad_right=0,
                    stride=2 ** 30, x_layout=c1g.LAYOUT_NLC),
               # w of 2^46 elements
               dict(N=1, C_in=2 ** 16, C_out=2 ** 30, T=1, K=1, pad_left=0, pad_right=0),
               dict(N=65536)):
        for dt in (c1g.C1G_F32, c1g.C1G_BF16):
            d = _desc(**dict(kw, dtype=dt))
            assert c1g.check(d) == 2, kw
            assert c1g.conv1d_workspace_size(d) == 0, kw
    lib = c1g.load_library()
    fake = ctypes.c_void_p(1 << 20)
    # N * C * L wraps to 0 in 64 bits
    for f in (lib.gn_apply, lib.gn_apply_bf16):
        assert f(2 ** 33, 2 ** 31, 1, 1, fake, fake, fake, None, None, fake, None) == 2
    assert lib.gn_apply(2 ** 20, 2 ** 12, 2 ** 12, 1, fake, fake, fake, None, None, fake,
                        None) == 2
    # N * G * slices wraps to 0 in 64 bits
    assert lib.c1g_gn_stats_workspace_size(2 ** 34, 2 ** 30, 2 ** 34, 2 ** 30) == 0
    assert lib.gn_stats(2 ** 34, 2 ** 30, 2 ** 34, 2 ** 30, 1e-5, fake, fake, fake, fake,
                        1 << 30, None) == 2


def test_log_names_plan_and_refusal():
    """C1G_LOG=1: every entry-point call writes one stderr line with its sizes,
    the plan and, for a refusal, the cause; without it nothing is written.
    (Refused calls only: nothing here reaches a launch.)"""
    import subprocess
    import sys
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import conv1d_implicit_gemm_amd as c1g
lib = c1g.load_library()
d = c1g.ConvDesc(2, 16, 32, 256, 3, 1, 1, 1, 1, 0, 0, 0)
P = None
bad_g = c1g.NormDesc(c1g.NORM_GROUP, 7, 1e-5, 0)
good = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
print(lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(bad_g), P, P, P, P, P, P, P, P, P, P, 0, P))
print(lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(good), P, P, P, P, P, P, P, P, P, P, 0, P))
f = ctypes.c_void_p(1 << 20)
print(lib.gn_apply(2 ** 33, 2 ** 31, 1, 1, f, f, f, P, P, f, P))
print(lib.conv1d_forward(ctypes.byref(c1g.ConvDesc(2, 16, 32, 256, 9, 1, 1, 4, 4, 0, 0, 0)), f, f, P, f, P, 0, P))
""" % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),)
    env = dict(os.environ, C1G_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["1", "1", "2", "2"]
    lines = [l for l in r.stderr.splitlines() if l.startswith("c1g: ")]
    assert len(lines) == 4, r.stderr
    assert lines[0].startswith("c1g: conv1d_gn_forward N=2 C_in=16 C_out=32 T=256 K=3")
    assert "G=7" in lines[0] and lines[0].endswith("invalid argument: G < 1 or C_out % G != 0")
    assert "| fused_single_pass T_out=256" in lines[1]
    assert lines[1].endswith("invalid argument: x, w or out is NULL")
    assert lines[2].startswith("c1g: gn_apply N=8589934592 C=2147483648 L=1 G=1")
    assert "unsupported configuration: N * C * L >= 2^32" in lines[2]
    assert lines[3].startswith("c1g: conv1d_forward") and "fp32: K > 8" in lines[3]
    env.pop("C1G_LOG")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0 and "c1g: " not in r.stderr


def test_force_path_split(monkeypatch):
    """C1G_FORCE_PATH=split: problems planned on a single-kernel route are
    planned on the split route (the workspace query follows); others keep
    their route."""
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    fused = _desc()
    persistent = _desc(C_in=64, C_out=256, T=1000, dtype=c1g.C1G_BF16)
    linear = _desc(N=64, C_in=256, C_out=512, T=1, K=1, pad_left=0, pad_right=0,
                   dtype=c1g.C1G_BF16)
    assert c1g.route(fused, gn) == "fused_single_pass"
    assert c1g.route(persistent, gn) == "fused_persistent"
    assert c1g.route(linear, gn) == "gemm_rows"
    monkeypatch.setenv("C1G_FORCE_PATH", "split")
    assert c1g.route(fused, gn) == "split"
    assert c1g.route(persistent, gn) == "split"
    assert c1g.route(linear, gn) == "gemm_rows"
    assert c1g.conv1d_gn_workspace_size(fused, gn) > 0
    monkeypatch.setenv("C1G_FORCE_PATH", "other")
    assert c1g.route(fused, gn) == "fused_single_pass"


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="needs a machine without a GPU, where every launch fails")
def test_launch_failure_is_reported_as_hip_error():
    """Where no device exists a call that passes validation fails at its
    launch: each entry point returns C1G_ERR_HIP, neither OK nor a crash.
    (Fake, aligned addresses: nothing reads them and nothing runs.)"""
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is present")
    lib = c1g.load_library()
    f = ctypes.c_void_p(1 << 20)
    d = _desc()
    gn = c1g.NormDesc(c1g.NORM_GROUP, 8, 1e-5, 0)
    assert c1g.route(d, gn) == "fused_single_pass"
    assert lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(gn), f, f, f, f, f, None, f, None,
                                 None, None, 0, None) == 5
    assert lib.conv1d_forward(ctypes.byref(d), f, f, None, f, f, 1 << 40, None) == 5
    assert lib.gn_stats(2, 32, 256, 8, 1e-5, f, f, f, f, 1 << 30, None) == 5
    assert lib.gn_apply(2, 32, 256, 8, f, f, f, None, None, f, None) == 5
    assert lib.gn_apply_bf16(2, 32, 256, 8, f, f, f, None, None, f, None) == 5


@pytest.mark.parametrize("K,stride,dilation,pad,T,tiles_t", [
    (5, 1, 2, (2, 2), 4096, 8),    # 512-position tiles: 4092 outputs
    (5, 2, 1, (2, 2), 8192, 8),    # stride 2: the 1027-row window of 512 positions does
                                   # not fit; interleaved passes (taps 0, 2, 4 and 1, 3),
                                   # each gathering every second row, do (514 rows)
    (6, 1, 1, (5, 0), 4096, 8),    # six taps: two passes of three on 512 positions
    (6, 1, 20, (0, 0), 4096, 16),  # six taps at dilation 20: a three-tap pass needs 552
                                   # rows, so 256 positions (356 rows); 3996 outputs
    (7, 1, 2, (12, 0), 4096, 8),   # seven taps: two passes (four and three) on 512
                                   # positions
    (7, 1, 11, (0, 0), 4096, 16),  # seven taps at dilation 11: a four-tap pass needs 545
                                   # rows, so 256 positions (322 rows); 4030 outputs
    (8, 1, 2, (7, 7), 4096, 8),    # eight taps: two passes of four on 512 positions
                                   # (518-row window each)
    (8, 1, 11, (0, 0), 4096, 32),  # eight taps at dilation 11: a four-tap pass needs 545
                                   # rows, so 128 positions (205 rows); 4019 outputs
    (4, 3, 1, (3, 0), 6000, 4),    # stride 3: three interleaved passes on 512 positions
                                   # (taps 0, 3 / 1 / 2; 513 rows); 2000 outputs
    (8, 4, 1, (2, 2), 16384, 8),   # stride 4: four interleaved passes of two taps (513 rows)
    (5, 5, 1, (0, 0), 20480, 8),   # stride 5: five interleaved passes of one tap (512 rows)
    (5, 2, 17, (0, 0), 8192, 32),  # stride 2 at dilation 17: an interleaved pass needs 546
                                   # rows and 256 positions 579, so 128 (323); 4062 outputs
])
def test_bf16_tile_choice(K, stride, dilation, pad, T, tiles_t):
    """The bf16 conv takes the largest tile (512, 256 or 128 positions) whose
    input window fits the LDS; the log's plan shows its position tiles.
    (Null pointers: the call is refused after planning.)"""
    import subprocess
    import sys
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import conv1d_implicit_gemm_amd as c1g
lib = c1g.load_library()
d = c1g.ConvDesc(4, 256, 1024, %d, %d, %d, %d, %d, %d, c1g.C1G_BF16, 0, 0)
nd = c1g.NormDesc(c1g.NORM_GROUP, 32, 1e-5, 0)
print(lib.conv1d_gn_forward(ctypes.byref(d), ctypes.byref(nd), *([None] * 10), 0, None))
""" % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))), T, K, stride, dilation,
       pad[0], pad[1])
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=dict(os.environ, C1G_LOG="1"), timeout=120)
    assert r.returncode == 0 and r.stdout.split() == ["1"], r.stderr
    line = [l for l in r.stderr.splitlines() if l.startswith("c1g: ")][0]
    assert "| fused_persistent" in line and " tiles=%dx8 " % tiles_t in line, line
    # the tile's positions and its passes over the input channels
    outs = (T + sum(pad) - dilation * (K - 1) - 1) // stride + 1
    tile = -(-outs // tiles_t)
    tile = 512 if tile > 256 else 256 if tile > 128 else 128
    passes = ""
    if tile == 512 and K > 5 and stride == 1:
        passes = " passes=2"
    elif tile == 512 and stride > 1:
        passes = " passes=%d interleaved" % min(stride, K)
    assert line.split(" -> ")[0].endswith(" tile=%d%s" % (tile, passes)), line
