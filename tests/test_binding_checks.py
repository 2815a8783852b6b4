"""CPU tests of the Python binding's argument checks: every tensor whose size
the kernels rely on is checked against the geometry before anything is
launched, so a wrong size raises ValueError instead of reaching the GPU.
The tensors here live on the CPU; shape checks run before the device check,
so each case fails on the CPU without touching a device."""
import pytest
import torch

import conv1d_implicit_gemm_amd as c1g

N, C_IN, C_OUT, T, K, G = 2, 16, 32, 64, 3, 8


def _xw():
    return torch.zeros(N, C_IN, T), torch.zeros(C_OUT, C_IN, K)


def _ch(n=C_OUT):
    return torch.zeros(n)


def _gn(**kw):
    x, w = _xw()
    args = dict(padding=1, norm="group", groups=G, gamma=_ch(), beta=_ch(), bias=_ch())
    args.update(kw)
    return c1g.conv1d_gn_forward(x, w, **args)


@pytest.mark.parametrize("name", ["bias", "gamma", "beta"])
def test_conv1d_gn_per_channel_short(name):
    with pytest.raises(ValueError, match=name):
        _gn(**{name: _ch(C_OUT - 1)})


def test_conv1d_gn_per_channel_2d():
    with pytest.raises(ValueError, match="gamma"):
        _gn(gamma=torch.zeros(1, C_OUT))


def test_conv1d_gn_rowmin_bias_short():
    with pytest.raises(ValueError, match="rowmin_bias"):
        _gn(rowmin_bias=_ch(C_OUT + 1))


def test_conv1d_gn_out_shape():
    with pytest.raises(ValueError, match="out"):
        _gn(out=torch.zeros(N, C_OUT, T - 1))


def test_conv1d_gn_c_in_mismatch():
    x = torch.zeros(N, C_IN + 1, T)
    w = torch.zeros(C_OUT, C_IN, K)
    with pytest.raises(ValueError, match="C_in"):
        c1g.conv1d_gn_forward(x, w, padding=1, groups=G)


def test_conv1d_gn_good_shapes_reach_device_check():
    # right sizes: the only complaint left is that the tensors are not on a GPU
    with pytest.raises(ValueError, match="device"):
        _gn()


def test_conv1d_forward_checks():
    x, w = _xw()
    with pytest.raises(ValueError, match="bias"):
        c1g.conv1d_forward(x, w, _ch(C_OUT - 2), padding=1)
    with pytest.raises(ValueError, match="out"):
        c1g.conv1d_forward(x, w, padding=1, out=torch.zeros(N, C_OUT + 1, T))
    with pytest.raises(ValueError, match="device"):
        c1g.conv1d_forward(x, w, _ch(), padding=1, out=torch.zeros(N, C_OUT, T))


def test_gn_apply_checks():
    y = torch.zeros(N, C_OUT, T)
    m, r = torch.zeros(N, G), torch.ones(N, G)
    with pytest.raises(ValueError, match="mean"):
        c1g.gn_apply(y, torch.zeros(N, G + 1), r, groups=G)
    with pytest.raises(ValueError, match="rstd"):
        c1g.gn_apply(y, m, torch.ones(N + 1, G))
    with pytest.raises(ValueError, match="groups"):
        c1g.gn_apply(y, torch.zeros(N, 5), torch.ones(N, 5))   # 32 % 5
    with pytest.raises(ValueError, match="gamma"):
        c1g.gn_apply(y, m, r, gamma=_ch(C_OUT // 2))
    with pytest.raises(ValueError, match="beta"):
        c1g.gn_apply(y, m, r, beta=_ch(C_OUT + 3))
    with pytest.raises(ValueError, match="out"):
        c1g.gn_apply(y, m, r, out=torch.zeros(N, C_OUT, T + 1))
    with pytest.raises(ValueError, match="mean"):
        c1g.gn_apply(y, torch.zeros(N * G), r)
    with pytest.raises(ValueError, match="device"):
        c1g.gn_apply(y, m, r, _ch(), _ch(), out=torch.zeros(N, C_OUT, T))


def test_gn_stats_checks():
    y = torch.zeros(N, C_OUT, T)
    with pytest.raises(ValueError, match="groups"):
        c1g.gn_stats(y, 5)
    with pytest.raises(ValueError, match="groups"):
        c1g.gn_stats(y, 0)
    with pytest.raises(ValueError, match="device"):
        c1g.gn_stats(y, G)


def test_prepared_checks():
    x, w = _xw()
    with pytest.raises(ValueError, match="mean"):
        c1g.PreparedConv1dGN(x, w, padding=1, norm="group", groups=G, mean=torch.zeros(N, 4))
    with pytest.raises(ValueError, match="rstd"):
        c1g.PreparedConv1dGN(x, w, padding=1, norm="layer_channels",
                             rstd=torch.zeros(N, G))                  # LN: [N, T_out]
    with pytest.raises(ValueError, match="gamma"):
        c1g.PreparedConv1dGN(x, w, padding=1, norm="group", groups=G, gamma=_ch(7))
    with pytest.raises(ValueError, match="out"):
        c1g.PreparedConv1dGN(x, w, padding=1, norm="group", groups=G,
                             out=torch.zeros(N, C_OUT, T + 2))
    with pytest.raises(ValueError, match="device"):
        c1g.PreparedConv1dGN(x, w, padding=1, norm="layer_channels",
                             mean=torch.zeros(N, T), rstd=torch.zeros(N, T))


@pytest.mark.parametrize("ws", [torch.zeros(64, 4).t(), [0] * 64])
def test_workspace_must_be_a_contiguous_tensor(ws):
    """A caller's workspace is checked before the device: a non-contiguous
    tensor, or something that is not a tensor, is refused."""
    x, w = _xw()
    with pytest.raises((ValueError, TypeError), match="workspace"):
        c1g.conv1d_forward(x, w, padding=1, workspace=ws)
    with pytest.raises((ValueError, TypeError), match="workspace"):
        _gn(workspace=ws)
