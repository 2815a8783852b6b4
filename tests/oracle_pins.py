"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each ``check_*`` takes a loaded ``oracle.Oracle`` and raises AssertionError on
a mismatch.  ``tests/test_oracle_pins.py`` runs them on the real build; the
mutation test runs them (in a subprocess, via ``python tests/oracle_pins.py
<lib>``) on copies of ``oracle.c`` with one planted mistake each and expects
at least one check to fail.

What pins what:
  * output length  -> the pages' stated lengths + a brute count of windows
  * conv index     -> the causal worked example of "Kimi-K2.6 l1_p5",
                      causality, the delta-kernel identity, an independently
                      written numpy brute force, torch float64 conv1d
  * GroupNorm      -> the invariant mean 0 / variance s2/(s2+eps) with unit
                      affine, the affine law, torch float64 group_norm
  * LN over C      -> the same invariant per (n,t), torch float64 layer_norm
  * row-min + bias -> out - bias2 constant over channels and equal to the min
  * k=1, T=1       -> numpy float64 X @ W^T
"""
from __future__ import annotations

import itertools
import os
import re
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


# ---------------------------------------------------------------- helpers
def _rng(seed):
    return np.random.default_rng(seed)


def brute_out_len(T, K, s, d, pl, pr):
    """Count the window starts t >= 0 whose last tap t*s + d*(K-1) still lies
    inside the padded signal of length T + pl + pr."""
    n = 0
    while n * s + d * (K - 1) <= T + pl + pr - 1:
        n += 1
    return n if n > 0 else -1


def brute_conv1d(x, w, bias, s, d, pl, pr):
    """Second, differently written convolution: materialise the zero-padded
    signal, gather each output's dilated window explicitly, dot with w."""
    N, C_in, T = x.shape
    C_out, _, K = w.shape
    xp = np.zeros((N, C_in, pl + T + pr))
    xp[:, :, pl:pl + T] = x
    T_out = brute_out_len(T, K, s, d, pl, pr)
    y = np.zeros((N, C_out, T_out))
    for t in range(T_out):
        idx = t * s + d * np.arange(K)
        win = xp[:, :, idx]                       # [N, C_in, K]
        y[:, :, t] = np.tensordot(win, w, axes=([1, 2], [1, 2]))
    if bias is not None:
        y += bias[None, :, None]
    return y


def _torch():
    import torch
    import torch.nn.functional as F
    return torch, F


# ---------------------------------------------------------------- checks
def check_out_len_pages(orc):
    """Lengths the pages state (tests/golden/out_len_cases.txt)."""
    with open(os.path.join(GOLDEN, "out_len_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            T, K, s, d, pl, pr, want = map(int, line.split())
            got = orc.out_len(T, K, s, d, pl, pr)
            assert got == want, (T, K, s, d, pl, pr, got, want)


def check_out_len_brute(orc):
    """Closed form vs brute window count over a grid of small geometries."""
    for T, K, s, d, pl, pr in itertools.product(
            [1, 2, 3, 7, 16, 31], [1, 2, 3, 4, 5], [1, 2, 3], [1, 2, 3], [0, 1, 2, 5], [0, 1, 3]):
        got = orc.out_len(T, K, s, d, pl, pr)
        want = brute_out_len(T, K, s, d, pl, pr)
        assert got == want, (T, K, s, d, pl, pr, got, want)


def check_causal_worked_example(orc):
    """The page's expansion of the first four causal outputs, exact in fp64
    (small integers keep every product and sum exact)."""
    terms = {}
    with open(os.path.join(GOLDEN, "causal_k4_worked_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            t, rhs = line.split(":")
            terms[int(t)] = [tuple(map(int, m)) for m in re.findall(r"w(\d+)\*x(\d+)", rhs)]
    rng = _rng(1)
    for trial in range(5):
        w = rng.integers(-9, 10, size=4).astype(np.float64)
        x = rng.integers(-9, 10, size=6).astype(np.float64)
        y = orc.conv1d(x[None, None, :], w[None, None, :], None, 1, 1, 3, 0)[0, 0]
        assert y.shape == (6,)
        for t, prods in terms.items():
            want = sum(w[j] * x[i] for j, i in prods)
            assert y[t] == want, (trial, t, y[t], want)


def check_causality(orc):
    """Perturbing inputs after t0 leaves every output at t <= t0 bit-identical."""
    rng = _rng(2)
    for K, d in [(4, 1), (3, 2), (5, 3)]:
        pl = (K - 1) * d
        x = rng.standard_normal((2, 3, 40))
        w = rng.standard_normal((4, 3, K))
        b = rng.standard_normal(4)
        y0 = orc.conv1d(x, w, b, 1, d, pl, 0)
        for t0 in [0, 5, 17, 38]:
            x2 = x.copy()
            x2[:, :, t0 + 1:] += rng.standard_normal(x2[:, :, t0 + 1:].shape) * 10
            y1 = orc.conv1d(x2, w, b, 1, d, pl, 0)
            assert np.array_equal(y0[:, :, :t0 + 1], y1[:, :, :t0 + 1]), (K, d, t0)
            if t0 + 1 < y0.shape[2]:
                assert not np.array_equal(y0[:, :, t0 + 1:], y1[:, :, t0 + 1:])


def check_delta_kernel(orc):
    """w[c,ci,j] = [c==ci][j==j0], no bias: y[n,c,t] = X(n,c,t*s+j0*d-pl) exactly."""
    rng = _rng(3)
    for (C, T, K, s, d, pl, pr) in [(3, 20, 4, 1, 1, 3, 0), (2, 17, 3, 2, 2, 1, 2),
                                    (4, 9, 5, 1, 3, 4, 4)]:
        x = rng.standard_normal((2, C, T))
        for j0 in range(K):
            w = np.zeros((C, C, K))
            for c in range(C):
                w[c, c, j0] = 1.0
            y = orc.conv1d(x, w, None, s, d, pl, pr)
            for t in range(y.shape[2]):
                u = t * s + j0 * d - pl
                want = x[:, :, u] if 0 <= u < T else np.zeros((2, C))
                assert np.array_equal(y[:, :, t], want), (C, T, K, s, d, j0, t)
    # causal with the newest tap selected is the identity
    x = rng.standard_normal((1, 3, 11))
    w = np.zeros((3, 3, 4))
    for c in range(3):
        w[c, c, 3] = 1.0
    assert np.array_equal(orc.conv1d(x, w, None, 1, 1, 3, 0), x)


def check_conv_brute(orc):
    """Loop oracle vs the gather-window brute force over small geometries."""
    rng = _rng(4)
    for (N, C_in, C_out, T, K, s, d, pl, pr) in itertools.product(
            [1, 2], [1, 3], [2, 4], [5, 12], [1, 2, 4], [1, 2], [1, 3], [0, 2], [0, 3]):
        if brute_out_len(T, K, s, d, pl, pr) < 1:
            continue
        x = rng.standard_normal((N, C_in, T))
        w = rng.standard_normal((C_out, C_in, K))
        b = rng.standard_normal(C_out)
        got = orc.conv1d(x, w, b, s, d, pl, pr)
        want = brute_conv1d(x, w, b, s, d, pl, pr)
        assert got.shape == want.shape, (got.shape, want.shape)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (N, C_in, C_out, T, K, s, d, pl, pr)


def check_conv_torch(orc):
    """Loop oracle vs torch float64 conv1d on an explicitly padded input."""
    torch, F = _torch()
    rng = _rng(5)
    for (N, C_in, C_out, T, K, s, d, pl, pr) in [
            (2, 16, 32, 64, 3, 1, 1, 1, 1), (1, 5, 7, 33, 4, 1, 1, 3, 0),
            (2, 8, 12, 50, 5, 1, 2, 2, 2), (3, 6, 4, 29, 3, 2, 1, 1, 1),
            (1, 9, 5, 40, 2, 3, 3, 0, 4), (4, 7, 6, 1, 1, 1, 1, 0, 0)]:
        x = rng.standard_normal((N, C_in, T))
        w = rng.standard_normal((C_out, C_in, K))
        b = rng.standard_normal(C_out)
        got = orc.conv1d(x, w, b, s, d, pl, pr)
        xt = F.pad(torch.from_numpy(x), (pl, pr))
        want = F.conv1d(xt, torch.from_numpy(w), torch.from_numpy(b), stride=s,
                        dilation=d).numpy()
        assert got.shape == want.shape
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (N, C_in, C_out, T, K, s, d)


def check_gemm_special_case(orc):
    """k=1, T=1: the convolution is X @ W^T."""
    rng = _rng(6)
    X = rng.standard_normal((9, 33))
    W = rng.standard_normal((20, 33))
    b = rng.standard_normal(20)
    got = orc.conv1d(X[:, :, None], W[:, :, None], b)[:, :, 0]
    assert np.allclose(got, X @ W.T + b, rtol=1e-12, atol=1e-12)


def _gn_cases():
    return [(2, 8, 30, 4), (3, 12, 7, 3), (1, 16, 1, 4), (2, 6, 5, 6), (2, 5, 9, 1)]


def check_group_norm_invariant(orc):
    """Unit affine: per (n,g) mean(z) = 0 and var(z) = s2/(s2+eps) with s2
    the population variance of the group's values (numpy, independent)."""
    rng = _rng(7)
    for (N, C, L, G) in _gn_cases():
        for eps in (1e-5, 0.5):
            y = rng.standard_normal((N, C, L)) * 3.0 + 1.7
            z, mean, rstd = orc.group_norm(y, G, eps)
            cpg = C // G
            for n in range(N):
                for g in range(G):
                    vals = y[n, g * cpg:(g + 1) * cpg, :].ravel()
                    zv = z[n, g * cpg:(g + 1) * cpg, :].ravel()
                    s2 = np.var(vals)
                    assert abs(np.mean(zv)) <= 1e-12, (N, C, L, G, n, g)
                    assert abs(np.var(zv) - s2 / (s2 + eps)) <= 1e-12 * max(1.0, s2 / (s2 + eps))
                    assert abs(mean[n, g] - np.mean(vals)) <= 1e-12 * max(1, abs(np.mean(vals)))
                    assert abs(rstd[n, g] - 1.0 / np.sqrt(s2 + eps)) <= 1e-12 * rstd[n, g]


def check_group_norm_affine(orc):
    """z(gamma, beta) = gamma[c] * z(1, 0) + beta[c] channelwise."""
    rng = _rng(8)
    for (N, C, L, G) in _gn_cases():
        y = rng.standard_normal((N, C, L))
        gam = rng.uniform(0.5, 1.5, C)
        bet = rng.standard_normal(C) * 0.1
        z0, _, _ = orc.group_norm(y, G, 1e-5)
        z1, _, _ = orc.group_norm(y, G, 1e-5, gam, bet)
        assert np.allclose(z1, z0 * gam[None, :, None] + bet[None, :, None], rtol=1e-12, atol=1e-13)


def check_group_norm_torch(orc):
    torch, F = _torch()
    rng = _rng(9)
    for (N, C, L, G) in _gn_cases():
        y = rng.standard_normal((N, C, L)) + 0.5
        gam = rng.uniform(0.5, 1.5, C)
        bet = rng.standard_normal(C) * 0.1
        z, _, _ = orc.group_norm(y, G, 1e-5, gam, bet)
        want = F.group_norm(torch.from_numpy(y), G, torch.from_numpy(gam),
                            torch.from_numpy(bet), 1e-5).numpy()
        assert np.allclose(z, want, rtol=1e-10, atol=1e-10), (N, C, L, G)


def check_layer_norm_invariant(orc):
    rng = _rng(10)
    for (N, C, L) in [(2, 8, 5), (1, 16, 3), (3, 5, 1)]:
        y = rng.standard_normal((N, C, L)) * 2.0 - 0.7
        z, mean, rstd = orc.layer_norm_channels(y, 1e-5)
        for n in range(N):
            for l in range(L):
                vals = y[n, :, l]
                s2 = np.var(vals)
                assert abs(np.mean(z[n, :, l])) <= 1e-12
                assert abs(np.var(z[n, :, l]) - s2 / (s2 + 1e-5)) <= 1e-12
                assert abs(mean[n, l] - np.mean(vals)) <= 1e-12 * max(1, abs(np.mean(vals)))


def check_layer_norm_torch(orc):
    torch, F = _torch()
    rng = _rng(11)
    for (N, C, L) in [(2, 8, 5), (1, 16, 3), (3, 5, 1)]:
        y = rng.standard_normal((N, C, L))
        gam = rng.uniform(0.5, 1.5, C)
        bet = rng.standard_normal(C) * 0.1
        z, _, _ = orc.layer_norm_channels(y, 1e-5, gam, bet)
        yt = torch.from_numpy(y).permute(0, 2, 1)
        want = F.layer_norm(yt, (C,), torch.from_numpy(gam), torch.from_numpy(bet),
                            1e-5).permute(0, 2, 1).numpy()
        assert np.allclose(z, want, rtol=1e-10, atol=1e-10), (N, C, L)


def check_rowmin_bias(orc):
    """out - bias2 is constant over channels and equals the channel minimum."""
    rng = _rng(12)
    for (N, C, L) in [(3, 16, 1), (2, 7, 5)]:
        z = rng.standard_normal((N, C, L))
        b2 = rng.standard_normal(C)
        out, m = orc.rowmin_bias(z, b2)
        zmin = z.min(axis=1)                      # numpy's own reduction
        assert np.array_equal(m, zmin)
        # one rounding of (min + bias2[c]) per element, same as numpy's add
        assert np.array_equal(out, zmin[:, None, :] + b2[None, :, None])
        d = out - b2[None, :, None]
        assert np.allclose(d, np.broadcast_to(d[:, :1, :], d.shape), rtol=0, atol=1e-15 * 8)


def check_rowmin_nan(orc):
    """A row holding a NaN (in the first, a middle or the last channel, or in
    every channel) has a NaN minimum, as PyTorch's min over a dimension gives
    (the reduction of the page's model); rows without one are unaffected."""
    torch, _ = _torch()
    rng = _rng(14)
    N, C, L = 2, 9, 6
    z = rng.standard_normal((N, C, L))
    z[0, 0, 1] = np.nan
    z[0, 4, 2] = np.nan
    z[1, C - 1, 3] = np.nan
    z[1, :, 5] = np.nan
    b2 = rng.standard_normal(C)
    out, m = orc.rowmin_bias(z, b2)
    want = torch.min(torch.from_numpy(z), dim=1)[0].numpy()
    assert np.array_equal(np.isnan(m), np.isnan(want))
    assert np.isnan(want).sum() == 4
    ok = ~np.isnan(want)
    assert np.array_equal(m[ok], want[ok])
    assert np.array_equal(np.isnan(out), np.broadcast_to(np.isnan(want)[:, None, :], out.shape))


def check_forward_composition(orc):
    """forward() = conv -> GN -> row-min + bias2 on a small k=1, T=1 case
    against numpy/torch float64 built independently."""
    torch, F = _torch()
    rng = _rng(13)
    X = rng.standard_normal((6, 32))
    W = rng.standard_normal((32, 32)) / np.sqrt(32)
    gam = rng.uniform(0.5, 1.5, 32)
    bet = rng.standard_normal(32) * 0.1
    b2 = rng.standard_normal(32)
    r = orc.forward(X[:, :, None], W[:, :, None], None, norm="group", G=2, eps=1e-5,
                    gamma=gam, beta=bet, bias2=b2)
    Y = torch.from_numpy(X @ W.T)
    Z = F.group_norm(Y, 2, torch.from_numpy(gam), torch.from_numpy(bet), 1e-5).numpy()
    want = Z.min(axis=1, keepdims=True) + b2[None, :]
    assert np.allclose(r["out"][:, :, 0], want, rtol=1e-10, atol=1e-10)


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]


def run_all(orc):
    """Run every check; return the names of the ones that failed."""
    failed = []
    for chk in ALL_CHECKS:
        try:
            chk(orc)
        except AssertionError:
            failed.append(chk.__name__)
    return failed


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    import oracle
    orc = oracle.Oracle(sys.argv[1])
    failed = run_all(orc)
    print("FAILED:" + ",".join(failed) if failed else "ALL-PASS")
    sys.exit(1 if failed else 0)
