"""conv1d_implicit_gemm_amd - MI355X (gfx950) conv1d -> GroupNorm.

A thin ctypes binding over the C ABI in ``include/conv1d_gn.h``
(``libconv1d_gn.so``, built by ``python -m conv1d_implicit_gemm_amd.build``).
It only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory (tensors passed by
``data_ptr()``) and the current HIP stream.  If the library is missing the
functions raise; there is no other implementation to fall back to.

Entry points (same names as the C ABI):
    conv1d_forward(x, w, bias=None, *, stride, padding/pad_left/pad_right, causal, dilation)
    conv1d_gn_forward(x, w, bias=None, *, ..., norm, groups, eps, gamma, beta,
                      rowmin_bias=None, return_stats=False)
    conv1d_gn_forward_noalloc(x, w, bias=None, *, out, ...)   (no workspace, no allocation)
    gn_stats(y, groups, eps)        -> (mean[N,G], rstd[N,G])
    gn_apply(y, mean, rstd, gamma, beta, groups, out=None)   (fp32, or bf16 -> gn_apply_bf16)
Outputs are fp32 unless ``out_dtype=torch.bfloat16`` (or a bf16 ``out``) is
given: values are computed in fp32 and rounded to nearest even on the store.
Host-only helpers: out_len, route, workspace sizes, check.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconv1d_gn.so")

C1G_F32, C1G_BF16 = 0, 1
LAYOUT_NCL, LAYOUT_NLC = 0, 1
NORM_NONE, NORM_GROUP, NORM_LAYER_CHANNELS = 0, 1, 2
EPI_NONE, EPI_ROWMIN_BIAS = 0, 1
FLAG_NO_PERSISTENT = 1
FLAG_ROWMIN_ONE_LAUNCH = 2
FLAG_COOPERATIVE = 4
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace missing or too small", 4: "misaligned pointer",
          5: "HIP runtime error at launch"}

# every symbol include/conv1d_gn.h declares
EXPORTS = ["c1g_out_len", "c1g_check", "c1g_conv1d_workspace_size", "conv1d_forward",
           "c1g_gn_stats_workspace_size", "gn_stats", "gn_apply", "gn_apply_bf16",
           "c1g_conv1d_gn_workspace_size", "conv1d_gn_forward", "conv1d_gn_forward_noalloc",
           "c1g_route", "c1g_status_string"]
# device scratch conv1d_gn_forward_noalloc holds per device (its largest workspace)
NOALLOC_SCRATCH_BYTES = 64 << 20


class ConvDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("C_in", ctypes.c_int64), ("C_out", ctypes.c_int64),
                ("T", ctypes.c_int64), ("K", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("dilation", ctypes.c_int32), ("pad_left", ctypes.c_int32),
                ("pad_right", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("x_layout", ctypes.c_int32)]


class NormDesc(ctypes.Structure):
    _fields_ = [("norm", ctypes.c_int32), ("G", ctypes.c_int32), ("eps", ctypes.c_float),
                ("epilogue", ctypes.c_int32), ("flags", ctypes.c_int32)]


class C1GError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, STATUS.get(status, "unknown"), status))


_lock = threading.Lock()
_lib = None


def load_library():
    """Load libconv1d_gn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libconv1d_gn.so is not built; run "
                               "`python -m conv1d_implicit_gemm_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PD, PN = ctypes.POINTER(ConvDesc), ctypes.POINTER(NormDesc)
        i64, i32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        lib.c1g_out_len.restype = i64
        lib.c1g_out_len.argtypes = [PD]
        lib.c1g_check.restype = ctypes.c_int
        lib.c1g_check.argtypes = [PD, PN, sz]
        lib.c1g_conv1d_workspace_size.restype = sz
        lib.c1g_conv1d_workspace_size.argtypes = [PD]
        lib.conv1d_forward.restype = ctypes.c_int
        lib.conv1d_forward.argtypes = [PD, P, P, P, P, P, sz, P]
        lib.c1g_gn_stats_workspace_size.restype = sz
        lib.c1g_gn_stats_workspace_size.argtypes = [i64, i64, i64, i32]
        lib.gn_stats.restype = ctypes.c_int
        lib.gn_stats.argtypes = [i64, i64, i64, i32, ctypes.c_float, P, P, P, P, sz, P]
        lib.gn_apply.restype = ctypes.c_int
        lib.gn_apply.argtypes = [i64, i64, i64, i32, P, P, P, P, P, P, P]
        lib.gn_apply_bf16.restype = ctypes.c_int
        lib.gn_apply_bf16.argtypes = [i64, i64, i64, i32, P, P, P, P, P, P, P]
        lib.c1g_conv1d_gn_workspace_size.restype = sz
        lib.c1g_conv1d_gn_workspace_size.argtypes = [PD, PN]
        lib.conv1d_gn_forward.restype = ctypes.c_int
        lib.conv1d_gn_forward.argtypes = [PD, PN, P, P, P, P, P, P, P, P, P, P, sz, P]
        lib.conv1d_gn_forward_noalloc.restype = ctypes.c_int
        lib.conv1d_gn_forward_noalloc.argtypes = [PD, PN, P, P, P, P, P, P, P, P, P, P]
        lib.c1g_route.restype = ctypes.c_char_p
        lib.c1g_route.argtypes = [PD, PN]
        lib.c1g_status_string.restype = ctypes.c_char_p
        lib.c1g_status_string.argtypes = [ctypes.c_int]
        _lib = lib
        return lib


# ----------------------------------------------------------------- helpers
def _pads(K, dilation, padding, pad_left, pad_right, causal):
    if causal:
        if pad_left is not None or pad_right is not None or padding:
            raise ValueError("causal=True fixes the padding")
        return (K - 1) * dilation, 0
    if pad_left is None and pad_right is None:
        return padding, padding
    return (pad_left if pad_left is not None else padding,
            pad_right if pad_right is not None else padding)


def make_desc(N, C_in, C_out, T, K, *, stride=1, dilation=1, padding=0, pad_left=None,
              pad_right=None, causal=False, dtype=C1G_F32, out_dtype=C1G_F32,
              x_layout=LAYOUT_NCL) -> ConvDesc:
    pl, pr = _pads(K, dilation, padding, pad_left, pad_right, causal)
    return ConvDesc(N, C_in, C_out, T, K, stride, dilation, pl, pr, dtype, out_dtype, x_layout)


_DT_CODE = {torch.float32: C1G_F32, torch.bfloat16: C1G_BF16}


def _out_dtype(out, out_dtype):
    """The output's torch dtype: that of ``out`` when given, else out_dtype."""
    dt = out.dtype if out is not None else out_dtype
    if dt not in _DT_CODE:
        raise TypeError("outputs must be float32 or bfloat16, got %s" % (dt,))
    return dt


def make_norm(norm=None, groups=0, eps=1e-5, rowmin=False, persistent=True,
              one_launch=False, cooperative=False) -> NormDesc:
    """persistent=False forbids kernels whose workgroups wait on each other
    (no "fused_persistent" route; they need every workgroup of a round
    resident at once).  one_launch=True asks for the "gemm_rows" GroupNorm +
    row-min as one such launch instead of a GEMM plus a broadcast kernel.
    cooperative=True launches those kernels through the runtime's cooperative
    launch, for callers that run other work on the device concurrently."""
    code = {None: NORM_NONE, "none": NORM_NONE, "group": NORM_GROUP,
            "layer_channels": NORM_LAYER_CHANNELS}[norm]
    return NormDesc(code, groups if code == NORM_GROUP else 0, eps,
                    EPI_ROWMIN_BIAS if rowmin else EPI_NONE,
                    (0 if persistent else FLAG_NO_PERSISTENT) |
                    (FLAG_ROWMIN_ONE_LAUNCH if one_launch else 0) |
                    (FLAG_COOPERATIVE if cooperative else 0))


def out_len(desc: ConvDesc) -> int:
    return int(load_library().c1g_out_len(ctypes.byref(desc)))


def route(desc: ConvDesc, norm: NormDesc = None) -> str:
    return load_library().c1g_route(ctypes.byref(desc),
                                    ctypes.byref(norm) if norm is not None else None).decode()


def check(desc: ConvDesc, norm: NormDesc = None, ws_bytes: int = 1 << 62) -> int:
    return int(load_library().c1g_check(ctypes.byref(desc),
                                        ctypes.byref(norm) if norm is not None else None,
                                        ws_bytes))


def conv1d_workspace_size(desc: ConvDesc) -> int:
    return int(load_library().c1g_conv1d_workspace_size(ctypes.byref(desc)))


def conv1d_gn_workspace_size(desc: ConvDesc, norm: NormDesc) -> int:
    return int(load_library().c1g_conv1d_gn_workspace_size(ctypes.byref(desc),
                                                           ctypes.byref(norm)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _shape(t, name, shape):
    """Shape check of an optional tensor argument, done before anything else
    is looked at (device, dtype), so a wrong size never reaches a kernel."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _per_channel(t, name, C):
    """A per-channel parameter: exactly C values (shape [C])."""
    _shape(t, name, (C,))


def _stats_shape(desc, nd, T_out, G):
    """Shape of exported mean/rstd: [N, G] (GroupNorm) or [N, T_out] (channel LayerNorm)."""
    return (desc.N, G) if nd.norm == NORM_GROUP else (desc.N, T_out)


def _workspace(ws, device=None):
    """A caller's workspace: a contiguous tensor (any dtype) on the call's
    device (checked once device is given); returns (ws, its size in bytes)."""
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a tensor")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if device is not None and ws.device != device:
        raise ValueError("workspace must be on %s" % device)
    return ws, ws.numel() * ws.element_size()


def _raise(status, where):
    if status != 0:
        raise C1GError(status, where)


def _conv_desc(x, w, stride, padding, pad_left, pad_right, causal, dilation,
               out_dtype=torch.float32, channels_last=False, out=None):
    """The conv descriptor from the shapes of x and w, and ``out`` checked
    against [N, C_out, T_out]; no device or dtype check yet.  Returns
    (desc, T_out)."""
    if not isinstance(x, torch.Tensor) or not isinstance(w, torch.Tensor):
        raise TypeError("x and w must be tensors")
    if x.dim() != 3 or w.dim() != 3:
        raise ValueError("x must be [N, C_in, T] ([N, T, C_in] with channels_last) and w "
                         "[C_out, C_in, K]")
    if channels_last:
        N, T, C_in = x.shape
    else:
        N, C_in, T = x.shape
    C_out, C_in_w, K = w.shape
    if C_in_w != C_in:
        raise ValueError("x and w disagree on C_in")
    dt = C1G_BF16 if x.dtype == torch.bfloat16 else C1G_F32
    desc = make_desc(N, C_in, C_out, T, K, stride=stride, dilation=dilation, padding=padding,
                     pad_left=pad_left, pad_right=pad_right, causal=causal, dtype=dt,
                     out_dtype=_DT_CODE[out_dtype],
                     x_layout=LAYOUT_NLC if channels_last else LAYOUT_NCL)
    T_out = int(load_library().c1g_out_len(ctypes.byref(desc)))
    if T_out < 1:
        _raise(1, "conv1d (output length)")
    _shape(out, "out", (N, C_out, T_out))
    return desc, T_out


def _conv_device(x, w):
    """Device, dtype and contiguity of x and w (after every shape check)."""
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, "x", None, x.device)
    _need(w, "w", x.dtype, x.device)


# ----------------------------------------------------------------- entry points
def conv1d_forward(x, w, bias=None, *, stride=1, padding=0, pad_left=None, pad_right=None,
                   causal=False, dilation=1, out=None, out_dtype=torch.float32,
                   channels_last=False, workspace=None):
    """y = conv1d(x, w) + bias, output [N, C_out, T_out] (fp32 or bf16); x is
    [N, C_in, T], or [N, T, C_in] with channels_last=True."""
    lib = load_library()
    odt = _out_dtype(out, out_dtype)
    _per_channel(bias, "bias", w.shape[0] if isinstance(w, torch.Tensor) else -1)
    desc, T_out = _conv_desc(x, w, stride, padding, pad_left, pad_right, causal, dilation,
                             odt, channels_last, out)
    _workspace(workspace)
    _conv_device(x, w)
    _need(bias, "bias", torch.float32, x.device)
    if out is None:
        out = torch.empty((desc.N, desc.C_out, T_out), device=x.device, dtype=odt)
    _need(out, "out", odt, x.device)
    ws_bytes = lib.c1g_conv1d_workspace_size(ctypes.byref(desc))
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, device=x.device, dtype=torch.uint8)
    workspace, ws_have = _workspace(workspace, x.device)
    st = lib.conv1d_forward(ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(bias), _ptr(out),
                            _ptr(workspace), ws_have, _stream(x.device))
    _raise(st, "conv1d_forward")
    return out


def conv1d_gn_forward(x, w, bias=None, *, stride=1, padding=0, pad_left=None, pad_right=None,
                      causal=False, dilation=1, norm="group", groups=1, eps=1e-5, gamma=None,
                      beta=None, rowmin_bias=None, return_stats=False, out=None,
                      out_dtype=torch.float32, persistent=True, one_launch=False,
                      cooperative=False, channels_last=False, workspace=None):
    """conv -> GroupNorm / LayerNorm over channels / none -> optional row-min + bias.

    x is [N, C_in, T], or [N, T, C_in] with channels_last=True.  Returns out
    [N, C_out, T_out] (fp32, or bf16 with out_dtype=torch.bfloat16 or a bf16
    ``out``), or (out, mean, rstd) with return_stats=True (fp32 mean/rstd
    [N, G] for GroupNorm, [N, T_out] for the channel LayerNorm)."""
    lib = load_library()
    odt = _out_dtype(out, out_dtype)
    C_out = w.shape[0] if isinstance(w, torch.Tensor) else -1
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta"), (rowmin_bias, "rowmin_bias")):
        _per_channel(t, nm, C_out)
    desc, T_out = _conv_desc(x, w, stride, padding, pad_left, pad_right, causal, dilation,
                             odt, channels_last, out)
    nd = make_norm(norm, groups, eps, rowmin_bias is not None, persistent, one_launch,
                   cooperative)
    _workspace(workspace)
    _conv_device(x, w)
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta"), (rowmin_bias, "rowmin_bias")):
        _need(t, nm, torch.float32, x.device)
    if out is None:
        out = torch.empty((desc.N, desc.C_out, T_out), device=x.device, dtype=odt)
    _need(out, "out", odt, x.device)
    mean = rstd = None
    if return_stats and nd.norm != NORM_NONE:
        shp = _stats_shape(desc, nd, T_out, groups)
        mean = torch.empty(shp, device=x.device, dtype=torch.float32)
        rstd = torch.empty(shp, device=x.device, dtype=torch.float32)
    ws_bytes = lib.c1g_conv1d_gn_workspace_size(ctypes.byref(desc), ctypes.byref(nd))
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, device=x.device, dtype=torch.uint8)
    workspace, ws_have = _workspace(workspace, x.device)
    st = lib.conv1d_gn_forward(ctypes.byref(desc), ctypes.byref(nd), _ptr(x), _ptr(w),
                               _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(rowmin_bias),
                               _ptr(out), _ptr(mean), _ptr(rstd), _ptr(workspace), ws_have,
                               _stream(x.device))
    _raise(st, "conv1d_gn_forward")
    return (out, mean, rstd) if return_stats else out


def conv1d_gn_forward_noalloc(x, w, bias=None, *, out, stride=1, padding=0, pad_left=None,
                              pad_right=None, causal=False, dilation=1, norm="group", groups=1,
                              eps=1e-5, gamma=None, beta=None, rowmin_bias=None, mean=None,
                              rstd=None, persistent=True, one_launch=False, cooperative=False,
                              channels_last=False):
    """conv1d_gn_forward without a workspace, for callers that cannot
    allocate: the library's own device scratch (NOALLOC_SCRATCH_BYTES per
    device) serves as the workspace, and nothing is allocated here either, so
    ``out`` (and, to export the statistics, ``mean``/``rstd``) must be given.
    Raises C1GError (workspace) when the problem needs a larger workspace.
    Calls on one device share the scratch: calls that overlap in time on one
    device race; calls on one stream are ordered."""
    lib = load_library()
    C_out = w.shape[0] if isinstance(w, torch.Tensor) else -1
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta"), (rowmin_bias, "rowmin_bias")):
        _per_channel(t, nm, C_out)
    if not isinstance(out, torch.Tensor):
        raise TypeError("out must be a tensor")
    odt = _out_dtype(out, None)
    desc, T_out = _conv_desc(x, w, stride, padding, pad_left, pad_right, causal, dilation,
                             odt, channels_last, out)
    nd = make_norm(norm, groups, eps, rowmin_bias is not None, persistent, one_launch,
                   cooperative)
    if mean is not None or rstd is not None:
        if nd.norm == NORM_NONE:
            raise ValueError("mean/rstd exports need a normalisation")
        shp = _stats_shape(desc, nd, T_out, groups)
        _shape(mean, "mean", shp)
        _shape(rstd, "rstd", shp)
    _conv_device(x, w)
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta"), (rowmin_bias, "rowmin_bias"),
                  (mean, "mean"), (rstd, "rstd")):
        _need(t, nm, torch.float32, x.device)
    _need(out, "out", odt, x.device)
    st = lib.conv1d_gn_forward_noalloc(ctypes.byref(desc), ctypes.byref(nd), _ptr(x), _ptr(w),
                                       _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(rowmin_bias),
                                       _ptr(out), _ptr(mean), _ptr(rstd), _stream(x.device))
    _raise(st, "conv1d_gn_forward_noalloc")
    return out


def gn_stats(y, groups, eps=1e-5):
    """GroupNorm statistics of y [N, C, L]: (mean[N,G], rstd[N,G])."""
    lib = load_library()
    if not isinstance(y, torch.Tensor) or y.dim() != 3:
        raise ValueError("y must be a [N, C, L] tensor")
    N, C, L = y.shape
    if not isinstance(groups, int) or groups < 1 or C % groups:
        raise ValueError("groups must be a positive divisor of C = %d" % C)
    if not y.is_cuda:
        raise ValueError("y must be a device tensor")
    _need(y, "y", torch.float32, y.device)
    mean = torch.empty((N, groups), device=y.device, dtype=torch.float32)
    rstd = torch.empty_like(mean)
    ws_bytes = lib.c1g_gn_stats_workspace_size(N, C, L, groups)
    ws = torch.empty(ws_bytes, device=y.device, dtype=torch.uint8) if ws_bytes else None
    st = lib.gn_stats(N, C, L, groups, eps, _ptr(y), _ptr(mean), _ptr(rstd), _ptr(ws), ws_bytes,
                      _stream(y.device))
    _raise(st, "gn_stats")
    return mean, rstd


def gn_apply(y, mean, rstd, gamma=None, beta=None, groups=None, out=None):
    """out = (y - mean) * rstd * gamma + beta with per-(n, group) statistics.
    y and out are both fp32 (gn_apply) or both bf16 (gn_apply_bf16).
    ``out=y`` normalises in place."""
    lib = load_library()
    if not isinstance(y, torch.Tensor) or y.dim() != 3:
        raise ValueError("y must be a [N, C, L] tensor")
    if not isinstance(mean, torch.Tensor) or not isinstance(rstd, torch.Tensor):
        raise TypeError("mean and rstd must be tensors")
    N, C, L = y.shape
    if mean.dim() != 2:
        raise ValueError("mean must be [N, G], got %s" % (tuple(mean.shape),))
    G = groups if groups is not None else mean.shape[1]
    if not isinstance(G, int) or G < 1 or C % G:
        raise ValueError("groups must be a positive divisor of C = %d" % C)
    _shape(mean, "mean", (N, G))
    _shape(rstd, "rstd", (N, G))
    _per_channel(gamma, "gamma", C)
    _per_channel(beta, "beta", C)
    _shape(out, "out", (N, C, L))
    if not y.is_cuda:
        raise ValueError("y must be a device tensor")
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    _need(y, "y", y.dtype, y.device)
    for t, nm in ((mean, "mean"), (rstd, "rstd"), (gamma, "gamma"), (beta, "beta")):
        _need(t, nm, torch.float32, y.device)
    if out is None:
        out = torch.empty_like(y)
    _need(out, "out", y.dtype, y.device)
    fn, name = ((lib.gn_apply, "gn_apply") if y.dtype == torch.float32
                else (lib.gn_apply_bf16, "gn_apply_bf16"))
    st = fn(N, C, L, G, _ptr(y), _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(beta), _ptr(out),
            _stream(y.device))
    _raise(st, name)
    return out


class PreparedConv1dGN:
    """conv1d_gn_forward with every argument marshalled once.

    Holds references to the tensors it was built from; each call enqueues the
    same work on the stream that was current at construction.  For tight
    loops (benchmarks, graph capture) where per-call validation in Python
    would dominate."""

    def __init__(self, x, w, bias=None, *, stride=1, padding=0, pad_left=None, pad_right=None,
                 causal=False, dilation=1, norm="group", groups=1, eps=1e-5, gamma=None,
                 beta=None, rowmin_bias=None, out=None, out_dtype=torch.float32, mean=None,
                 rstd=None, persistent=True, one_launch=False, cooperative=False,
                 channels_last=False):
        lib = load_library()
        odt = _out_dtype(out, out_dtype)
        C_out = w.shape[0] if isinstance(w, torch.Tensor) else -1
        for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta"),
                      (rowmin_bias, "rowmin_bias")):
            _per_channel(t, nm, C_out)
        self.norm = make_norm(norm, groups, eps, rowmin_bias is not None, persistent,
                              one_launch, cooperative)
        self.desc, self.T_out = _conv_desc(x, w, stride, padding, pad_left, pad_right, causal,
                                           dilation, odt, channels_last, out)
        if mean is not None or rstd is not None:
            if self.norm.norm == NORM_NONE:
                raise ValueError("mean/rstd exports need a normalisation")
            st_shape = _stats_shape(self.desc, self.norm, self.T_out, groups)
            _shape(mean, "mean", st_shape)
            _shape(rstd, "rstd", st_shape)
        _conv_device(x, w)
        for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta"),
                      (rowmin_bias, "rowmin_bias"), (mean, "mean"), (rstd, "rstd")):
            _need(t, nm, torch.float32, x.device)
        if out is None:
            out = torch.empty((self.desc.N, self.desc.C_out, self.T_out), device=x.device,
                              dtype=odt)
        _need(out, "out", odt, x.device)
        ws_bytes = lib.c1g_conv1d_gn_workspace_size(ctypes.byref(self.desc),
                                                   ctypes.byref(self.norm))
        self.workspace = (torch.empty(ws_bytes, device=x.device, dtype=torch.uint8)
                          if ws_bytes else None)
        self.route = route(self.desc, self.norm)
        self.out = out
        self._keep = (x, w, bias, gamma, beta, rowmin_bias, mean, rstd)
        self._fn = lib.conv1d_gn_forward
        self._args = (ctypes.byref(self.desc), ctypes.byref(self.norm), _ptr(x), _ptr(w),
                      _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(rowmin_bias), _ptr(out),
                      _ptr(mean), _ptr(rstd), _ptr(self.workspace), ws_bytes,
                      _stream(x.device))
        check_status = lib.c1g_check(ctypes.byref(self.desc), ctypes.byref(self.norm), ws_bytes)
        _raise(check_status, "PreparedConv1dGN")

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            _raise(st, "conv1d_gn_forward")
        return self.out
