"""The allocation-free forward (wanvae_resblock_forward_noalloc) against the
forward with a caller workspace, on the GPU, through the C ABI.

Two calls in a row on one device share the library's own workspace array;
the second runs a smaller input, so anything left from the first that it
read would show.  The bar is the bf16 one (max|diff| / max|ref| <= 2e-2) and,
since both calls run the same kernels on the same values, bitwise equality.
"""
import numpy as np
import pytest

from causal_convolution_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_pair(torch, wv, blk, w, seed):
    print(f"[noalloc] {w.desc}", flush=True)
    xd = gu.to_dev(wl.make_x_host(w, seed=seed), w.dtype)
    ref = blk.forward(xd)
    out = torch.full_like(ref, float("nan"))
    blk.forward_noalloc(xd, out)
    torch.cuda.synchronize()
    err = gu.rel_err(gu.to_host(out), gu.to_host(ref))
    same = bool(torch.equal(out, ref))
    tol = gu.TOL_BF16 if w.dtype == wl.BF16 else gu.TOL_F32
    gu.report(f"noalloc forward {w.name}", err, tol, f"bitwise==forward: {same}")
    assert err <= tol
    assert same


def test_noalloc_forward_matches_forward_twice():
    torch = gu.require_gpu()
    import causal_convolution_amd as wv
    # one parameter set, two extents: the second call is smaller than the first
    big = wl.custom("noalloc_big", wl.BF16, 1, 4, 19, 70, 192, 192)
    small = wl.custom("noalloc_small", wl.BF16, 1, 2, 7, 33, 192, 192)
    p = wl.make_params(big, seed=21)
    blk = wv.ResBlock.from_host(p, torch.bfloat16)
    _run_pair(torch, wv, blk, big, seed=21)
    _run_pair(torch, wv, blk, small, seed=22)
    # a 1x1x1-shortcut block and the fp32 path share the same array
    sc = wl.custom("noalloc_sc", wl.BF16, 1, 3, 12, 40, 384, 192)
    blk_sc = wv.ResBlock.from_host(wl.make_params(sc, seed=23), torch.bfloat16)
    _run_pair(torch, wv, blk_sc, sc, seed=23)
    c1 = wl.WORKLOADS["c1"]
    blk_f32 = wv.ResBlock.from_host(wl.make_params(c1, seed=0), torch.float32)
    _run_pair(torch, wv, blk_f32, c1, seed=0)
    assert wv.wait_giveups() == 0


def test_noalloc_rejects_blocks_beyond_its_array():
    torch = gu.require_gpu()
    import causal_convolution_amd as wv
    w = wl.custom("noalloc_over", wl.BF16, 1, 21, 90, 160, 384, 384)   # 464 MB of workspace
    blk = wv.ResBlock.from_host(wl.make_params(wl.custom("p", wl.BF16, 1, 1, 1, 1, 384, 384)),
                                torch.bfloat16)
    assert blk.workspace_size(w.n, w.t, w.h, w.w) > 64 << 20
    x = torch.zeros((w.n, w.t, w.h, w.w, w.cin), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 3.0)
    with pytest.raises(wv.WanVaeError) as e:
        blk.forward_noalloc(x, y)
    assert e.value.status == wv.ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())   # nothing was enqueued
