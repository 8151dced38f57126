"""Helpers shared by the GPU tests: device/host transfer, oracle blocks,
sampled output boxes and the parity measure."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from causal_convolution_amd import workloads

# parity bars, max|diff| / max|ref|: fp32 paths, and bf16 inputs with fp32 accumulation
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def torch():
    import torch as _t
    return _t


def require_gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a visible MI355X"
    import causal_convolution_amd as wv
    wv.lib()  # fails loudly if the HIP library is not built
    return t


def tdtype(dt):
    t = torch()
    return t.bfloat16 if dt == workloads.BF16 else t.float32


def to_dev(a, dt):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(tdtype(dt)).contiguous()


def to_host(x):
    return x.float().cpu().numpy()


def oracle_block(p):
    return oracle.Block(p["gamma1"], p["beta1"], p["wa"], p["ba"], p["gamma2"], p["beta2"],
                        p["wb"], p["bb"], p.get("ws"), p.get("bs"))


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    m = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (m if m > 0 else 1.0)


def pcc(got, ref):
    a = np.asarray(got, np.float64).ravel()
    b = np.asarray(ref, np.float64).ravel()
    if a.size < 2:
        return 1.0
    return float(np.corrcoef(a, b)[0, 1])


def report(name, err, tol, extra=""):
    print(f"[parity] {name}: max|d|/max|ref| = {err:.3e} (bar {tol:.0e}) {extra}", flush=True)
    sys.stdout.flush()


def sample_boxes(T, H, W, n_random=8, size=4, seed=0):
    """Output boxes (t0,t1,h0,h1,w0,w1): the 4 spatial corners and 4 edge
    midpoints at the first and the last frames, plus random interior boxes."""
    rng = np.random.default_rng(seed)
    st, sh, sw = min(size, T), min(size, H), min(size, W)
    hs = [0, max(H - sh, 0), max((H - sh) // 2, 0)]
    ws = [0, max(W - sw, 0), max((W - sw) // 2, 0)]
    spots = [(hs[0], ws[0]), (hs[0], ws[1]), (hs[1], ws[0]), (hs[1], ws[1]),
             (hs[0], ws[2]), (hs[1], ws[2]), (hs[2], ws[0]), (hs[2], ws[1])]
    boxes = []
    for t0 in sorted({0, max(T - st, 0)}):
        for (h0, w0) in spots:
            boxes.append((t0, t0 + st, h0, h0 + sh, w0, w0 + sw))
    for _ in range(n_random):
        t0 = int(rng.integers(0, T - st + 1))
        h0 = int(rng.integers(0, H - sh + 1))
        w0 = int(rng.integers(0, W - sw + 1))
        boxes.append((t0, t0 + st, h0, h0 + sh, w0, w0 + sw))
    return boxes


def branch_err(blk_o, x, got, ref):
    """Parity of the residual branch alone: (y - S(x)) against the oracle's
    (y - S(x)), relative to the branch's own largest value, with S the
    oracle's shortcut (x itself, or the 1x1x1 conv) of the exact input
    values.  The block output is the branch plus S(x) ("return residual +
    shortcut"), so with an identity shortcut max|y| is about max|x| and an
    error of the conv branch would otherwise be measured against x."""
    s = oracle.shortcut(blk_o, np.ascontiguousarray(x, np.float32)).astype(np.float64)
    return rel_err(np.asarray(got, np.float64) - s, np.asarray(ref, np.float64) - s)


def window_compare(blk_o, x_dev, y_dev, boxes):
    """(max rel error of the device output against the oracle over the
    boxes, PCC, max rel error of the residual branch y - S(x)), the oracle fed
    with the exact device input bits of each box's receptive field."""
    N, T, H, W, _ = x_dev.shape
    refs, gots, brs, bgs = [], [], [], []
    for box in boxes:
        reg = oracle.receptive_region(box, (T, H, W))
        xr = to_host(x_dev[:, reg[0]:reg[1], reg[2]:reg[3], reg[4]:reg[5]])
        ref = oracle.resblock_window(blk_o, xr, reg, (T, H, W), box)
        t0, t1, h0, h1, w0, w1 = box
        got = to_host(y_dev[:, t0:t1, h0:h1, w0:w1])
        s = oracle.shortcut(blk_o, to_host(x_dev[:, t0:t1, h0:h1, w0:w1])).astype(np.float64)
        refs.append(ref.ravel())
        gots.append(got.ravel())
        brs.append((ref - s).ravel())
        bgs.append((got - s).ravel())
    ref = np.concatenate(refs)
    got = np.concatenate(gots)
    return rel_err(got, ref), pcc(got, ref), rel_err(np.concatenate(bgs), np.concatenate(brs))
