"""Independent host references used to pin the oracle (not the oracle itself).

* ``brute_conv``: a direct causal 3x3x3 convolution written as explicit
  Python loops with per-tap bounds checks (tiny inputs only).
* ``torch_*``: the same operations assembled from PyTorch CPU library
  routines in float64: ``F.normalize`` (the routine the Wan RMS_norm is
  written with, "Closing the gap", section 4), ``F.silu``, ``F.pad`` and
  ``F.conv3d`` (channels-first, weight [C_out, C_in, kD, kH, kW]).

Neither shares code with ``oracle/oracle.c``.
"""
from __future__ import annotations

import math

import numpy as np


def brute_conv(x, w, bias=None, cache=None):
    """Direct causal conv, float64 result (no rounding).

    x [N,T,H,W,Cin], w [Cout,Cin,3,3,3], cache [N,2,H,W,Cin] or None.
    Output (t,h,w) reads input (t+kt-2, h+kh-1, w+kw-1); frames before 0 come
    from the cache (frame -2 = cache[:,0], frame -1 = cache[:,1]) or are 0;
    rows/columns outside the image are 0.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    N, T, H, W, Cin = x.shape
    Cout = w.shape[0]
    y = np.zeros((N, T, H, W, Cout))
    for n in range(N):
        for t in range(T):
            for h in range(H):
                for ww in range(W):
                    for co in range(Cout):
                        s = 0.0
                        for kt in range(3):
                            for kh in range(3):
                                for kw in range(3):
                                    ts, hs, ws = t + kt - 2, h + kh - 1, ww + kw - 1
                                    if hs < 0 or hs >= H or ws < 0 or ws >= W:
                                        continue
                                    if ts < 0:
                                        if cache is None:
                                            continue
                                        src = np.asarray(cache, np.float64)[n, ts + 2, hs, ws]
                                    else:
                                        src = x[n, ts, hs, ws]
                                    for ci in range(Cin):
                                        s += w[co, ci, kt, kh, kw] * src[ci]
                        if bias is not None:
                            s += float(bias[co])
                        y[n, t, h, ww, co] = s
    return y


def torch_conv(z, w, bias=None, cache=None):
    """Causal conv through F.pad + F.conv3d in float64, channels-last in/out."""
    import torch
    import torch.nn.functional as F
    zc = torch.as_tensor(np.asarray(z, np.float64)).permute(0, 4, 1, 2, 3)
    if cache is not None:
        cc = torch.as_tensor(np.asarray(cache, np.float64)).permute(0, 4, 1, 2, 3)
        zc = F.pad(torch.cat([cc, zc], dim=2), (1, 1, 1, 1, 0, 0))
    else:
        zc = F.pad(zc, (1, 1, 1, 1, 2, 0))
    wt = torch.as_tensor(np.asarray(w, np.float64))
    bt = None if bias is None else torch.as_tensor(np.asarray(bias, np.float64))
    return F.conv3d(zc, wt, bt).permute(0, 2, 3, 4, 1).numpy()


def torch_norm(x, gamma, beta=None, eps=1e-12):
    """Wan RMS_norm as F.normalize over channels * sqrt(C) * gamma + beta (float64)."""
    import torch
    import torch.nn.functional as F
    xt = torch.as_tensor(np.asarray(x, np.float64))
    C = xt.shape[-1]
    u = F.normalize(xt, p=2.0, dim=-1, eps=eps) * math.sqrt(C) * torch.as_tensor(
        np.asarray(gamma, np.float64))
    if beta is not None:
        u = u + torch.as_tensor(np.asarray(beta, np.float64))
    return u.numpy()


def torch_silu(u):
    import torch
    import torch.nn.functional as F
    return F.silu(torch.as_tensor(np.asarray(u, np.float64))).numpy()


def f32(a):
    return np.asarray(a, np.float64).astype(np.float32)


def torch_block(p, x, cache_a=None, cache_b=None):
    """ResidualBlock from library routines, rounding to float32 where the
    oracle stores (n1, a, n2, y).  Returns y and the conv inputs n1, n2."""
    n1 = f32(torch_silu(torch_norm(x, p["gamma1"], p["beta1"])))
    a = f32(torch_conv(n1, p["wa"], p["ba"], cache_a))
    n2 = f32(torch_silu(torch_norm(a, p["gamma2"], p["beta2"])))
    acc = torch_conv(n2, p["wb"], p["bb"], cache_b)
    if p.get("ws") is None:
        sc = np.asarray(x, np.float64)
    else:
        sc = np.einsum("nthwc,oc->nthwo", np.asarray(x, np.float64),
                       np.asarray(p["ws"], np.float64)) + np.asarray(p["bs"], np.float64)
    return f32(acc + sc), n1, n2


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.max(np.abs(ref)) if ref.size else 0.0
    if m == 0.0:
        return float(np.max(np.abs(got - ref))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / m)
