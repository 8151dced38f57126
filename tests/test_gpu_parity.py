"""GPU parity: every entry point of libwanvae.so against the CPU oracle.

Inputs are seeded; bf16 tensors are compared on the exact bf16 values the
device holds (widened to float32 for the oracle).  Bars (max|diff| /
max|ref|): 1e-5 for fp32 paths, 2e-2 for bf16-in / fp32-accumulate paths.

Small shapes are compared element by element over the whole output; they
span several workgroup tiles (8 rows x 32 columns x up to 192 channels) and
have ragged tails in H, W and the row count.  The five full-size workloads
run in the launch configuration the benchmark times and are compared on
sampled output boxes (corners, edge midpoints, first and last frames,
random interior), each computed by the oracle from its receptive field.
"""
import math

import numpy as np
import pytest

import oracle
from causal_convolution_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def wv(torch):
    import causal_convolution_amd as m
    return m


@pytest.fixture(autouse=True)
def no_wait_giveups(wv):
    """Every test leaves the conv's bounded flag waits untouched: a wait that
    reached its bound means a launch left its synchronisation protocol and
    its output cannot be trusted, whatever the parity check said."""
    wv.wait_giveups_reset()
    yield
    n = wv.wait_giveups()
    assert n == 0, f"{n} bounded flag waits gave up during the test"


def rnd(rng, shape, scale=1.0, dt=wl.F32):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return wl.round_bf16(a) if dt == wl.BF16 else a


def tol(dt):
    return gu.TOL_BF16 if dt == wl.BF16 else gu.TOL_F32


# --------------------------------------------------------------------------- norm
@pytest.mark.parametrize("dt", [wl.F32, wl.BF16])
# 544 and 992: one row per 16-lane group with a partly used last run (odd
# multiples of 32 above 512); 1024: the widest row
@pytest.mark.parametrize("C", [32, 64, 96, 192, 384, 544, 992, 1024])
@pytest.mark.parametrize("rows", [1, 17, 70001])
def test_rmsnorm_silu(torch, wv, dt, C, rows):
    rng = np.random.default_rng(C * 1000 + rows)
    x = rnd(rng, (rows, C), 2.0, dt)
    g = rng.uniform(0.5, 1.5, C).astype(np.float32)
    b = rnd(rng, (C,), 0.3)
    ref = oracle.norm_silu(x, g, b)
    xd = gu.to_dev(x, dt)
    y = wv.rmsnorm_silu(xd, gu.to_dev(g, wl.F32), gu.to_dev(b, wl.F32))
    err = gu.rel_err(gu.to_host(y), ref)
    gu.report(f"norm {dt} C={C} rows={rows}", err, tol(dt))
    assert err <= tol(dt)
    # in place, and beta = NULL
    ref0 = oracle.norm_silu(x, g, None)
    wv.rmsnorm_silu(xd, gu.to_dev(g, wl.F32), None, out=xd)
    assert gu.rel_err(gu.to_host(xd), ref0) <= tol(dt)


def test_rmsnorm_silu_zero_rows_and_vectors(torch, wv):
    C = 96
    g = gu.to_dev(np.ones(C, np.float32), wl.F32)
    b_h = np.linspace(-2, 2, C).astype(np.float32)
    x = torch.zeros((5, C), dtype=torch.bfloat16, device="cuda")
    y = wv.rmsnorm_silu(x, g, gu.to_dev(b_h, wl.F32))
    ref = oracle.norm_silu(np.zeros((5, C), np.float32), np.ones(C, np.float32), b_h)
    assert gu.rel_err(gu.to_host(y), ref) <= gu.TOL_BF16
    e = torch.zeros((0, C), dtype=torch.bfloat16, device="cuda")
    assert wv.rmsnorm_silu(e, g, None).shape == (0, C)


# --------------------------------------------------------------------------- conv
CONV_SHAPES = [
    # N, T, H, W, Cin, Cout
    (1, 3, 19, 70, 64, 96),      # ragged H (19 = 2*8+3) and W (70 = 2*32+6)
    (2, 4, 9, 33, 96, 192),      # batch 2, W one past a tile
    (1, 5, 8, 32, 384, 384),     # exact tiles, 2 channel blocks
    (1, 3, 17, 40, 192, 128),
    (1, 2, 5, 7, 32, 32),        # smaller than one tile
    (1, 1, 1, 1, 32, 64),        # one position, one frame
    (1, 4, 3, 35, 1024, 1024),   # widest channel count
    (1, 3, 6, 36, 160, 224),     # channel counts with odd multiples of 32
    # image heights for which the 18-row tiles are chosen (exact and ragged)
    (1, 3, 36, 40, 64, 128),     # 2 x 18 rows, 64-channel blocks
    (2, 2, 35, 33, 96, 96),      # 35 rows: one 18-row tile padded by one row; Cout 96
    (1, 4, 18, 64, 192, 192),    # one 18-row tile, 3 channel blocks
    # C_out a multiple of 96 but not 64: 12-row tiles of 96 channels
    (1, 2, 13, 40, 96, 288),     # 3 channel blocks, ragged H (13 = 12 + 1) and W
    (1, 3, 24, 32, 32, 96),      # exact tiles, smallest input slice count
    (1, 3, 14, 40, 48, 96),      # 3 input slices: odd stage counts (9 with a cache) end on a lone stage
    (2, 4, 13, 33, 112, 288),    # 7 input slices, 3 channel blocks, batch 2, ragged H and W
    # the decoder's head and tail: 16 latent channels in (conv_in), 3 out (conv_out)
    (1, 3, 10, 40, 16, 384),     # one 16-channel stage per temporal tap
    (1, 3, 12, 40, 96, 3),       # C_out padded to one 32-channel block, 2-byte stores
    (2, 2, 9, 33, 16, 3),        # both at once, batch 2
    (1, 2, 5, 35, 32, 40),       # a partial second channel block (40 = 32 + 8)
    (1, 2, 6, 33, 48, 100),      # C_out % 8 != 0 (rows not 16-byte aligned)
    # C_out <= 3: the taps-as-rows kernel (8 x 62 output tiles, chunks of 27 frames)
    (1, 30, 9, 70, 32, 3),       # two frame chunks, ragged rows and columns
    (1, 2, 17, 64, 96, 1),       # one output channel, 3 row tiles
    (2, 3, 8, 62, 48, 2),        # two output channels, exact tiles, batch 2
]


@pytest.mark.parametrize("shape", CONV_SHAPES)
@pytest.mark.parametrize("with_cache", [False, True])
def test_causal_conv3d_bf16(torch, wv, shape, with_cache):
    N, T, H, W, Cin, Cout = shape
    rng = np.random.default_rng(sum(shape) + with_cache)
    x = rnd(rng, (N, T, H, W, Cin), 1.0, wl.BF16)
    w = rnd(rng, (Cout, Cin, 3, 3, 3), 1 / math.sqrt(27 * Cin), wl.BF16)
    b = rnd(rng, (Cout,), 0.1)
    cache = rnd(rng, (N, 2, H, W, Cin), 1.0, wl.BF16) if with_cache else None
    ref = oracle.causal_conv3d(x, w, b, cache)
    y = wv.causal_conv3d(gu.to_dev(x, wl.BF16), wv.pack_conv3d_weights(gu.to_dev(w, wl.BF16)),
                         gu.to_dev(b, wl.F32),
                         None if cache is None else gu.to_dev(cache, wl.BF16))
    err = gu.rel_err(gu.to_host(y), ref)
    gu.report(f"conv bf16 {shape} cache={with_cache}", err, gu.TOL_BF16, f"pcc={gu.pcc(gu.to_host(y), ref):.6f}")
    assert err <= gu.TOL_BF16


def test_wait_giveups_are_counted(torch, wv):
    """A bound of zero polls, set from the host, makes the conv's flag waits
    give up at once: every launch still runs to completion (its result is
    then meaningless), and the give-ups are counted.  With the default bound
    the same conv counts none and matches the oracle."""
    rng = np.random.default_rng(5)
    shape = (1, 3, 19, 70, 64, 96)
    N, T, H, W, Cin, Cout = shape
    x = rnd(rng, (N, T, H, W, Cin), 1.0, wl.BF16)
    w = rnd(rng, (Cout, Cin, 3, 3, 3), 1 / math.sqrt(27 * Cin), wl.BF16)
    xd, pw = gu.to_dev(x, wl.BF16), wv.pack_conv3d_weights(gu.to_dev(w, wl.BF16))
    wv.set_wait_bound(0)
    try:
        wv.causal_conv3d(xd, pw)
        n = wv.wait_giveups()
    finally:
        wv.set_wait_bound(-1)
    print(f"[giveups] bound 0: {n} waits gave up", flush=True)
    assert n > 0
    wv.wait_giveups_reset()
    y = wv.causal_conv3d(xd, pw)
    assert wv.wait_giveups() == 0
    assert gu.rel_err(gu.to_host(y), oracle.causal_conv3d(x, w)) <= gu.TOL_BF16


@pytest.mark.parametrize("shape", [(1, 4, 16, 16, 64, 64), (2, 3, 5, 7, 3, 5), (1, 2, 9, 4, 33, 1)])
@pytest.mark.parametrize("with_cache", [False, True])
def test_causal_conv3d_f32(torch, wv, shape, with_cache):
    N, T, H, W, Cin, Cout = shape
    rng = np.random.default_rng(sum(shape) + 7 * with_cache)
    x = rnd(rng, (N, T, H, W, Cin))
    w = rnd(rng, (Cout, Cin, 3, 3, 3), 1 / math.sqrt(27 * Cin))
    b = rnd(rng, (Cout,), 0.1)
    cache = rnd(rng, (N, 2, H, W, Cin)) if with_cache else None
    ref = oracle.causal_conv3d(x, w, b, cache)
    y = wv.causal_conv3d(gu.to_dev(x, wl.F32), wv.pack_conv3d_weights(gu.to_dev(w, wl.F32)),
                         gu.to_dev(b, wl.F32), None if cache is None else gu.to_dev(cache, wl.F32))
    err = gu.rel_err(gu.to_host(y), ref)
    gu.report(f"conv f32 {shape} cache={with_cache}", err, gu.TOL_F32)
    assert err <= gu.TOL_F32


def test_causal_conv3d_no_bias_and_empty(torch, wv):
    rng = np.random.default_rng(3)
    x = rnd(rng, (1, 2, 8, 32, 64), 1.0, wl.BF16)
    w = rnd(rng, (32, 64, 3, 3, 3), 0.05, wl.BF16)
    pw = wv.pack_conv3d_weights(gu.to_dev(w, wl.BF16))
    y = wv.causal_conv3d(gu.to_dev(x, wl.BF16), pw)
    assert gu.rel_err(gu.to_host(y), oracle.causal_conv3d(x, w)) <= gu.TOL_BF16
    e = torch.zeros((1, 0, 8, 32, 64), dtype=torch.bfloat16, device="cuda")
    assert wv.causal_conv3d(e, pw).shape == (1, 0, 8, 32, 32)


@pytest.mark.parametrize("cin,cout,dtype", [(16, 1, wl.BF16), (16, 3, wl.BF16), (48, 96, wl.BF16),
                                            (96, 40, wl.BF16), (384, 192, wl.BF16),
                                            (3, 5, wl.F32), (64, 33, wl.F32)])
def test_pack_conv3d_weights_layout(torch, wv, cin, cout, dtype):
    """The packed order is the one the header documents, element for element
    (a pure permutation: compared bit for bit)."""
    rng = np.random.default_rng(cin * 1000 + cout)
    w = rnd(rng, (cout, cin, 3, 3, 3), 1.0, dtype)
    got = gu.to_host(wv.pack_conv3d_weights(gu.to_dev(w, dtype)).data)
    taps = w.reshape(cout, cin, 27)
    if dtype == wl.BF16:
        # [kt][cin/16][kh*3+kw][cout_p][16], cout_p = cout rounded up to 32, zero padding
        cout_p = (cout + 31) // 32 * 32
        taps = np.concatenate([taps, np.zeros((cout_p - cout, cin, 27), taps.dtype)])
        want = taps.reshape(cout_p, cin // 16, 16, 3, 9).transpose(3, 1, 4, 0, 2).reshape(-1)
    else:
        # [cout][kt*9+kh*3+kw][cin]
        want = taps.transpose(0, 2, 1).reshape(-1)
    assert got.shape == want.shape
    assert np.array_equal(got.astype(np.float32), want.astype(np.float32))


# --------------------------------------------------------------------------- pointwise
@pytest.mark.parametrize("dt", [wl.F32, wl.BF16])
@pytest.mark.parametrize("cin,cout", [(16, 16), (16, 3), (64, 48), (1, 1)])
@pytest.mark.parametrize("rows", [1, 1000, 70001])
def test_pointwise_conv(torch, wv, dt, cin, cout, rows):
    """1x1x1 conv (the decoder's post_quant_conv, 16 -> 16) against the oracle."""
    rng = np.random.default_rng(cin * 7 + cout * 3 + rows)
    x = rnd(rng, (rows, cin), 1.0, dt)
    w = rnd(rng, (cout, cin), 1 / math.sqrt(cin), dt)
    b = rnd(rng, (cout,), 0.1)
    ref = oracle.pointwise_conv(x, w, b)
    y = wv.pointwise_conv(gu.to_dev(x, dt), gu.to_dev(w, dt), gu.to_dev(b, wl.F32))
    err = gu.rel_err(gu.to_host(y), ref)
    gu.report(f"pointwise {dt} {cin}->{cout} rows={rows}", err, tol(dt))
    assert err <= tol(dt)
    y0 = wv.pointwise_conv(gu.to_dev(x, dt), gu.to_dev(w, dt), None)
    assert gu.rel_err(gu.to_host(y0), oracle.pointwise_conv(x, w, None)) <= tol(dt)


# --------------------------------------------------------------------------- block, small
SMALL_BLOCKS = [
    wl.custom("id96", wl.BF16, 1, 4, 19, 70, 96, 96),
    wl.custom("sc384_192", wl.BF16, 1, 3, 12, 40, 384, 192),
    wl.custom("id192_b2", wl.BF16, 2, 3, 9, 33, 192, 192),
    wl.custom("sc64_128", wl.BF16, 1, 5, 8, 64, 64, 128),
    wl.custom("f32_sc", wl.F32, 1, 3, 6, 10, 64, 32),
    # 18-row tiles: identity and 1x1x1-shortcut epilogues, 64- and 96-channel tiles
    wl.custom("id128_h36", wl.BF16, 1, 3, 36, 40, 128, 128),
    wl.custom("sc192_96_h35", wl.BF16, 1, 3, 35, 40, 192, 96),
    wl.custom("sc96_288", wl.BF16, 1, 3, 13, 36, 96, 288),   # 96-channel tiles, 3 blocks, shortcut
    # a wide odd channel count (norm rows cut raggedly) with norm tiles crossing frames
    wl.custom("sc544_32", wl.BF16, 1, 3, 5, 37, 544, 32),
    # 1x1x1 shortcuts on the projection GEMM: a 64-wide last channel chunk, a
    # single 64-wide chunk, and ragged position tiles
    wl.custom("sc256_320", wl.BF16, 1, 3, 7, 45, 256, 320),
    wl.custom("sc128_64", wl.BF16, 2, 2, 9, 20, 128, 64),
    # conv A with norm2 + SiLU in its epilogue (out_dim 96 or 32): ragged rows
    # and columns, batch 2, and with the fused 1x1x1 shortcut
    wl.custom("id96_b2", wl.BF16, 2, 5, 13, 37, 96, 96),
    wl.custom("id32", wl.BF16, 1, 4, 17, 45, 32, 32),
    wl.custom("sc64_96", wl.BF16, 1, 3, 12, 40, 64, 96),
    # the identity residual through the ring with 32-channel tiles over
    # several channel blocks (160 = 5 x 32)
    wl.custom("id160", wl.BF16, 1, 3, 10, 40, 160, 160),
    # the identity residual with 96-channel tiles over three channel blocks,
    # ragged rows and columns
    wl.custom("id288", wl.BF16, 1, 3, 13, 36, 288, 288),
    # 24 frames, 96 channels: the convs' tiles go in frame super-blocks of 20
    # groups, the last one ragged (23 groups: 20 + 3)
    wl.custom("id96_t24", wl.BF16, 1, 24, 13, 40, 96, 96),
    # the same on the 32-channel tiles (norm2 in conv A's epilogue), and with
    # the fused 1x1x1 shortcut stages on the 96-channel tiles (21 groups)
    wl.custom("id32_t24", wl.BF16, 1, 24, 9, 40, 32, 32),
    wl.custom("sc64_96_t22", wl.BF16, 1, 22, 12, 40, 64, 96),
]


def _block(wv, w, seed=0):
    p = wl.make_params(w, seed)
    return p, wv.ResBlock.from_host(p, gu.tdtype(w.dtype))


def test_block_c1_full(torch, wv):
    w = wl.WORKLOADS["c1"]
    p, blk = _block(wv, w)
    x = wl.make_x_host(w)
    ref = oracle.resblock_full(gu.oracle_block(p), x)
    y = blk.forward(gu.to_dev(x, w.dtype))
    err = gu.rel_err(gu.to_host(y), ref)
    eb = gu.branch_err(gu.oracle_block(p), x, gu.to_host(y), ref)
    gu.report("block c1 fp32 full", err, gu.TOL_F32, f"branch y-x: {eb:.3e}")
    assert err <= gu.TOL_F32
    assert eb <= gu.TOL_F32


@pytest.mark.parametrize("w", SMALL_BLOCKS, ids=lambda w: w.name)
def test_block_small_full_and_stream(torch, wv, w):
    p, blk = _block(wv, w, seed=5)
    x = wl.make_x_host(w, seed=5)
    ref = oracle.resblock_full(gu.oracle_block(p), x)
    xd = gu.to_dev(x, w.dtype)
    y = blk.forward(xd)
    err = gu.rel_err(gu.to_host(y), ref)
    eb = gu.branch_err(gu.oracle_block(p), x, gu.to_host(y), ref)
    gu.report(f"block {w.name} full", err, tol(w.dtype),
              f"branch y-S(x): {eb:.3e} pcc={gu.pcc(gu.to_host(y), ref):.6f}")
    assert err <= tol(w.dtype)
    assert eb <= tol(w.dtype)
    # chunks of 1, 2 and 3 frames (3 leaves a shorter last chunk for T = 4, 5)
    for ts in (1, 2, 3):
        ca, cb = blk.new_caches(w.n, w.h, w.w)
        ys = [blk.stream_step(xd[:, t0:t0 + ts].contiguous(), ca, cb) for t0 in range(0, w.t, ts)]
        ys = torch.cat(ys, dim=1)
        e2 = gu.rel_err(gu.to_host(ys), ref)
        same = bool(torch.equal(ys, y))
        gu.report(f"block {w.name} stream t_step={ts}", e2, tol(w.dtype), f"bitwise==full: {same}")
        assert e2 <= tol(w.dtype)
        # the same kernels add the same terms in the same order; a cache of
        # zeros only adds exact zeros where full-T skips the causal pad
        assert same, f"stream with chunks of {ts} differs from full-T"
        assert e2 <= tol(w.dtype)


# --------------------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_block_full_size_sampled(torch, wv, name):
    w = wl.WORKLOADS[name]
    print(f"[full-size] {name}: {w.desc}", flush=True)
    p, blk = _block(wv, w)
    x = wl.make_x_device(w)
    y = blk.forward(x)
    torch.cuda.synchronize()
    # 16 boxes at the corners and edge midpoints of the first and last frames,
    # 120 at random: 136 boxes of 4 x 4 x 4 outputs
    boxes = gu.sample_boxes(w.t, w.h, w.w, n_random=120)
    err, r, eb = gu.window_compare(gu.oracle_block(p), x, y, boxes)
    gu.report(f"block {name} full-size, {len(boxes)} boxes", err, tol(w.dtype),
              f"branch y-S(x): {eb:.3e} pcc={r:.6f}")
    assert err <= tol(w.dtype)
    assert eb <= tol(w.dtype)
    del x, y, blk
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_block_c2_full_output(torch, wv):
    """The latent-resolution block [1,21,90,160,384] compared over its whole
    output: the oracle runs the clip in chunks of 3 frames with its caches
    (its streamed result equals its full-T result bit for bit), printing as
    it goes."""
    w = wl.WORKLOADS["c2"]
    p, blk = _block(wv, w)
    x = wl.make_x_device(w)
    y = gu.to_host(blk.forward(x))
    xh = gu.to_host(x)
    del x
    torch.cuda.empty_cache()
    ob = gu.oracle_block(p)
    ca = np.zeros((w.n, 2, w.h, w.w, w.cin), np.float32)
    cb = np.zeros((w.n, 2, w.h, w.w, w.cout), np.float32)
    ref = np.empty_like(y)
    for t0 in range(0, w.t, 3):
        ref[:, t0:t0 + 3] = oracle.resblock_stream_step(ob, np.ascontiguousarray(xh[:, t0:t0 + 3]), ca, cb)
        print(f"[c2 full] oracle frames {t0}..{min(t0 + 3, w.t) - 1} done", flush=True)
    err = gu.rel_err(y, ref)
    eb = gu.branch_err(ob, xh, y, ref)
    gu.report("block c2 full output", err, gu.TOL_BF16, f"branch y-x: {eb:.3e} pcc={gu.pcc(y, ref):.6f}")
    assert err <= gu.TOL_BF16
    assert eb <= gu.TOL_BF16


def test_c5_stream_equals_full_t(torch, wv):
    w = wl.WORKLOADS["c5"]
    p, blk = _block(wv, w)
    x = wl.make_x_device(w)
    y = blk.forward(x)
    ca, cb = blk.new_caches(w.n, w.h, w.w)
    ws = blk.workspace(w.n, 1, w.h, w.w)
    ys = torch.empty_like(y)
    for t in range(w.t):
        blk.stream_step(x[:, t:t + 1], ca, cb, out=ys[:, t:t + 1], workspace=ws)
    torch.cuda.synchronize()
    diff = (ys.float() - y.float()).abs().max().item()
    scale = y.float().abs().max().item()
    same = bool(torch.equal(ys, y))
    gu.report("c5 stream (41 x T=1) vs full-T", diff / scale, gu.TOL_BF16, f"bitwise: {same}")
    assert diff / scale <= gu.TOL_BF16
    assert same, "c5 streamed frame by frame differs from full-T"
    # and the streamed output against the oracle on sampled boxes
    boxes = gu.sample_boxes(w.t, w.h, w.w, n_random=16)
    err, _, eb = gu.window_compare(gu.oracle_block(p), x, ys, boxes)
    gu.report(f"c5 stream vs oracle, {len(boxes)} boxes", err, gu.TOL_BF16, f"branch y-S(x): {eb:.3e}")
    assert err <= gu.TOL_BF16
    assert eb <= gu.TOL_BF16
    del x, y, ys
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- robustness
def test_deterministic_and_workspace_independent(torch, wv):
    w = wl.custom("det", wl.BF16, 1, 5, 20, 64, 192, 96)
    p, blk = _block(wv, w, seed=9)
    xd = gu.to_dev(wl.make_x_host(w, seed=9), w.dtype)
    ws = blk.workspace(w.n, w.t, w.h, w.w)
    y1 = blk.forward(xd, workspace=ws)
    ws.view(torch.int16).fill_(-1)          # 0xffff bf16 = NaN everywhere
    y2 = blk.forward(xd, workspace=ws)
    assert torch.equal(y1, y2)


def test_output_guard_bands(torch, wv):
    w = wl.custom("guard", wl.BF16, 1, 3, 10, 40, 96, 96)
    p, blk = _block(wv, w, seed=11)
    xd = gu.to_dev(wl.make_x_host(w, seed=11), w.dtype)
    n = w.positions * w.cout
    g = 4096
    buf = torch.full((n + 2 * g,), 7.0, dtype=torch.bfloat16, device="cuda")
    y = buf[g:g + n].view(w.n, w.t, w.h, w.w, w.cout)
    blk.forward(xd, out=y)
    torch.cuda.synchronize()
    assert bool((buf[:g] == 7.0).all()) and bool((buf[g + n:] == 7.0).all())
    assert torch.equal(y, blk.forward(xd))


@pytest.mark.parametrize("cout,norms", [(192, 2), (96, 1)])
def test_timing_counts_launches(torch, wv, cout, norms):
    """Launches per forward: norm1, conv A, norm2, conv B; with 96 (or 32)
    output channels conv A computes norm2 in its epilogue, one norm less."""
    w = wl.custom("timing", wl.BF16, 1, 2, 8, 32, cout, cout)
    p, blk = _block(wv, w)
    xd = gu.to_dev(wl.make_x_host(w), w.dtype)
    wv.timing_reset()
    wv.timing_enable(True)
    blk.forward(xd)
    blk.forward(xd)
    wv.timing_enable(False)
    n_norm, ms_norm = wv.timing_read(wv.KERNEL_NORM)
    n_conv, ms_conv = wv.timing_read(wv.KERNEL_CONV_BF16)
    wv.timing_reset()
    assert n_norm == 2 * norms and n_conv == 4
    assert ms_norm > 0 and ms_conv > 0


# --------------------------------------------------------------------------- attention
def _attn_check(torch, wv, x_host, p, label, frames=None, nq=None, seed=0):
    """Run the attention block on x and compare with the oracle: the whole
    output and, separately, the attention branch y - x (which the residual
    would otherwise dwarf); on full-size inputs only sampled queries of some
    frames."""
    blk = wv.AttentionBlock.from_host(p)
    xd = gu.to_dev(x_host, wl.BF16)
    y = gu.to_host(blk.forward(xd))
    args = (p["gamma"], p["beta"], p["wqkv"], p["bqkv"], p["wo"], p["bo"])
    N, T, H, W, C_ = x_host.shape
    if frames is None:
        ref = oracle.attention_block(x_host, *args)
        got, xs = y, x_host
    else:
        rng = np.random.default_rng(seed)
        refs, gots, xss = [], [], []
        for (n, t) in frames:
            q = np.unique(np.concatenate([[0, W - 1, (H - 1) * W, H * W - 1],
                                          rng.integers(0, H * W, size=nq)]))
            refs.append(oracle.attention_block(x_host, *args, frame=(n, t), queries=q))
            gots.append(y[n, t].reshape(-1, C_)[q])
            xss.append(x_host[n, t].reshape(-1, C_)[q])
        ref, got, xs = np.concatenate(refs), np.concatenate(gots), np.concatenate(xss)
    err = gu.rel_err(got, ref)
    err_branch = gu.rel_err(got - xs, ref - xs)
    gu.report(f"attention {label}", err, gu.TOL_BF16, f"branch y-x: {err_branch:.3e} pcc={gu.pcc(got - xs, ref - xs):.6f}")
    assert err <= gu.TOL_BF16
    assert err_branch <= gu.TOL_BF16


@pytest.mark.parametrize("shape", [
    (1, 2, 5, 7, 64),      # 35 positions: one query block, a ragged second key block
    (1, 1, 12, 13, 128),   # 156 positions: 2 query blocks, 5 key blocks
    (2, 2, 9, 16, 384),    # the decoder's width, batch 2
    (1, 1, 17, 31, 384),   # 527 positions: ragged query and key blocks
    (1, 2, 1, 1, 64),      # one position per frame: o = v
])
def test_attention_block_small(torch, wv, shape):
    rng = np.random.default_rng(sum(shape))
    x = wl.round_bf16(rng.standard_normal(shape).astype(np.float32))
    p = wl.make_attention_params(shape[-1], seed=sum(shape))
    _attn_check(torch, wv, x, p, f"{shape}")


def test_attention_block_growing_scores(torch, wv):
    """Scores that keep growing along the key sequence: the positions of the
    frame turn from one direction v toward another, u, and the q and k
    projections are a scaled identity, so a late query scores the later keys
    ever higher and its running maximum passes the softmax reference by more
    than 2^8 again and again (the kernel's rescale path, which random inputs
    reach only at the first key block)."""
    C, H, W = 128, 16, 40
    HW = H * W
    rng = np.random.default_rng(11)
    a0, a1 = rng.standard_normal(C), rng.standard_normal(C)
    u = a0 / np.linalg.norm(a0)
    v = a1 - (a1 @ u) * u
    v /= np.linalg.norm(v)
    u, v = u * np.sqrt(C), v * np.sqrt(C)   # unit RMS
    theta = np.linspace(np.pi / 2, 0.0, HW)
    x = wl.round_bf16((np.cos(theta)[:, None] * u + np.sin(theta)[:, None] * v).astype(np.float32))
    x = x.reshape(1, 1, H, W, C)
    p = wl.make_attention_params(C, seed=11)
    p["gamma"][:] = 1.0
    p["beta"][:] = 0.0
    s = np.sqrt(3.5)
    eye = wl.round_bf16((s * np.eye(C)).astype(np.float32))
    p["wqkv"][:C] = eye
    p["wqkv"][C:2 * C] = eye
    p["bqkv"][:2 * C] = 0.0
    # precondition of the data: the last query's running maximum (log2 units,
    # keys in blocks of 32) passes the reference by more than 8 several times
    xf = x.reshape(HW, C).astype(np.float64)
    xn = xf / np.sqrt((xf * xf).mean(axis=1, keepdims=True))
    sc = (s * s) * (xn @ xn[-1]) / np.sqrt(C) * np.log2(np.e)
    ref_max, moves = -np.inf, 0
    for j in range(0, HW, 32):
        m = sc[j:j + 32].max()
        if m > ref_max + 8.0:
            ref_max, moves = m, moves + 1
    assert moves >= 5, moves
    _attn_check(torch, wv, x, p, f"growing scores, {moves} reference moves")


def test_attention_block_latent_sampled(torch, wv):
    """The latent-resolution mid-block, [1, 21, 90, 160, 384], on sampled
    queries (corners and random positions) of the first, a middle and the
    last frame; the oracle computes k and v of each sampled frame in full."""
    w = wl.custom("attn", wl.BF16, 1, 21, 90, 160, 384, 384)
    xd = wl.make_x_device(w, seed=3)
    x = xd.float().cpu().numpy()
    del xd
    p = wl.make_attention_params(384, seed=3)
    _attn_check(torch, wv, x, p, "latent [1,21,90,160,384] sampled", frames=[(0, 0), (0, 10), (0, 20)],
                nq=24, seed=3)
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- upsampler
def _upsample_check(torch, wv, xd, x_host, w, b, label, frames=None, rows=None):
    """upsample2d_conv on the device input xd against the oracle on x_host
    (the same values): the whole output, or the given output rows of the
    given frames (x_host then holds just those frames, in that order)."""
    wp = wv.pack_conv2d_weights(torch.from_numpy(w).to("cuda").to(torch.bfloat16))
    y = wv.upsample2d_conv(xd, wp, torch.from_numpy(b).to("cuda"))
    torch.cuda.synchronize()
    if frames is None:
        got = gu.to_host(y)
        ref = oracle.upsample2d_conv(x_host, w, b)
    else:
        got, ref = [], []
        for (r0, r1) in rows:
            ref.append(oracle.upsample2d_conv(x_host, w, b, frames=[(0, i) for i in range(len(frames))],
                                              rows=(r0, r1)))
            got.append(np.stack([gu.to_host(y[n, t, r0:r1]) for (n, t) in frames]))
        got, ref = np.concatenate(got, axis=1), np.concatenate(ref, axis=1)
    del y
    err = gu.rel_err(got, ref)
    gu.report(f"upsample2d {label}", err, gu.TOL_BF16, f"pcc={gu.pcc(got, ref):.6f}")
    assert err <= gu.TOL_BF16


@pytest.mark.parametrize("shape,cout", [
    ((1, 2, 5, 17, 16), 32),     # 10 x 34 out: ragged row and column tiles, one 32-channel block
    ((1, 3, 9, 16, 64), 64),     # 18-row tiles
    ((2, 1, 7, 20, 384), 192),   # the decoder's 384 -> 192, batch 2
    ((1, 2, 6, 12, 192), 96),    # C_out a multiple of 96: by output phase
    ((1, 2, 13, 33, 96), 96),    # by phase: 13 input rows (12-row tiles + 1), 33 columns (32 + 1)
    ((2, 1, 12, 32, 192), 192),  # by phase: exact tiles, two channel blocks, batch 2
    ((1, 3, 25, 70, 48), 96),    # by phase: 3 input slices (a lone last stage), ragged rows and columns
    ((1, 1, 1, 1, 96), 96),      # by phase: one input position, a 2 x 2 output
    ((1, 2, 5, 9, 64), 288),     # by phase: three 96-channel blocks
    ((2, 1, 7, 40, 16), 96),     # by phase: one input slice (a lone stage per tile), batch 2
    ((1, 2, 4, 9, 96), 40),      # a padded channel block
    ((1, 1, 1, 1, 32), 3),       # one input position, 3 output channels (2-byte stores)
])
def test_upsample2d_small(torch, wv, shape, cout):
    rng = np.random.default_rng(sum(shape) + cout)
    x = wl.round_bf16(rng.standard_normal(shape).astype(np.float32))
    w, b = wl.make_upsample_params(shape[-1], cout, seed=sum(shape))
    _upsample_check(torch, wv, gu.to_dev(x, wl.BF16), x, w, b, f"{shape} -> {cout}")


@pytest.mark.parametrize("shape,cout", [
    ((1, 21, 90, 160, 384), 192),    # after the latent-resolution up block
    ((1, 81, 360, 640, 192), 96),    # the last upsampler, to 720 x 1280 (output 14 GB)
])
def test_upsample2d_decoder_sampled(torch, wv, shape, cout):
    """Decoder-size upsamplers: the first, a middle and the last frame, the
    output rows at the top and bottom edges and in the middle."""
    n, t, h, w_, cin = shape
    xd = wl.make_x_device(wl.custom("up", wl.BF16, n, t, h, w_, cin, cout), seed=5)
    frames = [(0, 0), (0, t // 2), (0, t - 1)]
    x_host = np.stack([xd[0, tt].float().cpu().numpy() for (_, tt) in frames])[None]
    w, b = wl.make_upsample_params(cin, cout, seed=5)
    H2 = 2 * h
    rows = [(0, 3), (H2 // 2 - 1, H2 // 2 + 2), (H2 - 3, H2)]
    _upsample_check(torch, wv, xd, x_host, w, b, f"{shape} -> {cout} sampled", frames=frames, rows=rows)
    del xd
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- reference copy
@pytest.mark.parametrize("nbytes", [16, 16 * 1000, (1 << 22) + 48])
def test_stream_copy(torch, wv, nbytes):
    """The measurement copy moves every byte and nothing past the end."""
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    for unroll in (1, 2, 4, 8):
        buf = torch.full((nbytes + 4096,), 7, dtype=torch.uint8, device="cuda")
        wv.stream_copy(src, buf[:nbytes], unroll, 4)
        torch.cuda.synchronize()
        assert torch.equal(buf[:nbytes], src)
        assert bool((buf[nbytes:] == 7).all())


# --------------------------------------------------------------------------- stream state
@pytest.mark.parametrize("C", [16, 96, 384])
def test_stream_cache_layout(torch, wv, C):
    """export / import convert between the cache's 16-channel slices,
    [n][2][C/16][h][w][16], and channels-last [n][2][h][w][C], bit for bit."""
    n, h, w = 2, 5, 7
    g = torch.Generator(device="cuda").manual_seed(C)
    frames = torch.randn((n, 2, h, w, C), device="cuda", generator=g).to(torch.bfloat16)
    sliced = frames.view(n, 2, h, w, C // 16, 16).permute(0, 1, 4, 2, 3, 5).contiguous().view(-1)
    got = wv.export_stream_cache(sliced, n, h, w, C)
    assert torch.equal(got, frames)
    back = torch.zeros_like(sliced)
    wv.import_stream_cache(frames, back)
    assert torch.equal(back, sliced)


@pytest.mark.parametrize("w", [wl.custom("ckpt_sc", wl.BF16, 1, 6, 12, 40, 384, 192),
                               wl.custom("ckpt_id96", wl.BF16, 2, 6, 13, 37, 96, 96),
                               wl.custom("ckpt_f32", wl.F32, 1, 6, 6, 10, 64, 32)],
                         ids=lambda w: w.name)
def test_stream_checkpoint_resume(torch, wv, w):
    """Save the stream state mid-clip and resume from it: after 3 frames the
    caches go to the host channels-last, the device caches are discarded, new
    ones are set from the saved frames, and the last 3 frames stream on.  The
    result equals full-T bit for bit, and the saved frames equal the oracle's
    caches after the same 3 frames (n1 and n2 of frames 1 and 2) within the
    bar."""
    p, blk = _block(wv, w, seed=31)
    x = wl.make_x_host(w, seed=31)
    xd = gu.to_dev(x, w.dtype)
    full = blk.forward(xd)
    ca, cb = blk.new_caches(w.n, w.h, w.w)
    ys = [blk.stream_step(xd[:, t:t + 1].contiguous(), ca, cb) for t in range(3)]
    saved_a = blk.export_cache(ca, w.n, w.h, w.w, w.cin).cpu()
    saved_b = blk.export_cache(cb, w.n, w.h, w.w, w.cout).cpu()
    del ca, cb
    ca, cb = blk.new_caches(w.n, w.h, w.w)
    blk.import_cache(saved_a.to("cuda"), ca)
    blk.import_cache(saved_b.to("cuda"), cb)
    ys += [blk.stream_step(xd[:, t:t + 1].contiguous(), ca, cb) for t in range(3, w.t)]
    ys = torch.cat(ys, 1)
    assert torch.equal(ys, full), "resumed stream differs from full-T"
    # the saved state against the oracle's caches after the same frames
    ob = gu.oracle_block(p)
    oa = np.zeros((w.n, 2, w.h, w.w, w.cin), np.float32)
    obb = np.zeros((w.n, 2, w.h, w.w, w.cout), np.float32)
    oracle.resblock_stream_step(ob, np.ascontiguousarray(x[:, :3]), oa, obb)
    ea = gu.rel_err(saved_a.float().numpy(), oa)
    eb = gu.rel_err(saved_b.float().numpy(), obb)
    gu.report(f"checkpoint {w.name}: saved cache_a / cache_b vs oracle", max(ea, eb), tol(w.dtype),
              f"a {ea:.3e} b {eb:.3e}")
    assert ea <= tol(w.dtype) and eb <= tol(w.dtype)


@pytest.mark.parametrize("cout", [96, 192])
def test_block_zero_conv_a(torch, wv, cout):
    """Conv A's weight and bias all zero: every a vector is zero, the norm's
    clamp takes over and n2 = silu(beta2) at every position (in conv A's
    epilogue at 96 channels, in the norm kernel at 192); the pad positions
    conv B reads stay 0.  Against the oracle, with the residual branch gated
    on its own."""
    w = wl.custom(f"zero_a_{cout}", wl.BF16, 1, 3, 13, 37, cout, cout)
    p = wl.make_params(w, seed=41)
    p["wa"][:] = 0.0
    p["ba"][:] = 0.0
    blk = wv.ResBlock.from_host(p, torch.bfloat16)
    # the branch is small here (conv B of one constant vector), so x is scaled
    # by 2^-5 (exactly, in bf16) to keep y's own rounding, which grows with
    # |y| ~ |x|, small next to the branch
    x = wl.make_x_host(w, seed=41) * np.float32(2.0 ** -5)
    y = gu.to_host(blk.forward(gu.to_dev(x, w.dtype)))
    ob = gu.oracle_block(p)
    ref = oracle.resblock_full(ob, x)
    err = gu.rel_err(y, ref)
    eb = gu.branch_err(ob, x, y, ref)
    gu.report(f"block zero conv A, {cout} channels", err, gu.TOL_BF16, f"branch y-x: {eb:.3e}")
    assert err <= gu.TOL_BF16 and eb <= gu.TOL_BF16


# --------------------------------------------------------------------------- upsample3d
@pytest.mark.parametrize("shape,cout", [
    ((1, 3, 5, 17, 16), 32),     # 5 output frames, ragged row and column tiles
    ((2, 2, 9, 16, 64), 64),     # batch 2, 18-row tiles
    ((1, 4, 6, 12, 192), 96),    # 96-channel (kh-outer) tiles, 7 output frames
    ((1, 1, 2, 3, 32), 3),       # one input frame: one output frame, 3 output channels
    ((1, 3, 4, 9, 96), 40),      # a padded channel block
])
def test_upsample3d_small(torch, wv, shape, cout):
    """The whole output against the oracle; and bitwise equal to upsample2d
    of the frames doubled after the first (the same kernel on the same
    values, the frame read remapped)."""
    rng = np.random.default_rng(sum(shape) + 2 * cout)
    x = wl.round_bf16(rng.standard_normal(shape).astype(np.float32))
    w, b = wl.make_upsample_params(shape[-1], cout, seed=sum(shape) + 1)
    wp = wv.pack_conv2d_weights(torch.from_numpy(w).to("cuda").to(torch.bfloat16))
    bd = torch.from_numpy(b).to("cuda")
    xd = gu.to_dev(x, wl.BF16)
    y = wv.upsample3d_conv(xd, wp, bd)
    ref = oracle.upsample3d_conv(x, w, b)
    got = gu.to_host(y)
    err = gu.rel_err(got, ref)
    gu.report(f"upsample3d {shape} -> {cout}", err, gu.TOL_BF16, f"pcc={gu.pcc(got, ref):.6f}")
    assert got.shape == ref.shape and err <= gu.TOL_BF16
    idx = torch.tensor([0] + [k for k in range(1, shape[1]) for _ in range(2)], device="cuda")
    y2 = wv.upsample2d_conv(xd.index_select(1, idx).contiguous(), wp, bd)
    assert torch.equal(y, y2)


def test_upsample3d_decoder_sampled(torch, wv):
    """up_blocks[0]'s upsample3d at the decoder's shape, [1,21,90,160,384] ->
    [1,41,180,320,192]: output frames 0..4 against the oracle on input frames
    0..2 and output frames 37..40 against it on input frames 18..20 (an
    output frame reads no later input frame, and frames 2k - 1, 2k only input
    frame k), rows at the top, middle and bottom."""
    w_ = wl.custom("up3", wl.BF16, 1, 21, 90, 160, 384, 192)
    xd = wl.make_x_device(w_, seed=7)
    w, b = wl.make_upsample_params(384, 192, seed=7)
    wp = wv.pack_conv2d_weights(torch.from_numpy(w).to("cuda").to(torch.bfloat16))
    y = wv.upsample3d_conv(xd, wp, torch.from_numpy(b).to("cuda"))
    torch.cuda.synchronize()
    rows = [(0, 3), (89, 92), (177, 180)]
    errs = []
    for (i0, i1, o0) in [(0, 3, 0), (18, 21, 36)]:
        ref = oracle.upsample3d_conv(gu.to_host(xd[:, i0:i1]), w, b)      # 5 output frames
        # a clip starting at input frame i0 reproduces output frames 2 i0 + 1 .. (not 2 i0 - 1, 2 i0)
        first = 0 if i0 == 0 else 1
        for (r0, r1) in rows:
            got = gu.to_host(y[:, o0 + first:o0 + 5, r0:r1])
            errs.append(gu.rel_err(got, ref[:, first:, r0:r1]))
    err = max(errs)
    gu.report("upsample3d [1,21,90,160,384] -> 192 sampled", err, gu.TOL_BF16)
    assert err <= gu.TOL_BF16
    del xd, y
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- decoder tail, fused
TAIL_SHAPES = [
    (1, 3, 12, 40, 96, 3),       # the decoder's 96 -> 3, ragged W
    (2, 2, 9, 33, 16, 3),        # one 16-channel slice, batch 2
    (1, 30, 9, 70, 32, 3),       # two frame chunks, ragged rows and columns
    (1, 2, 17, 64, 96, 1),       # one output channel, 3 row tiles
    (2, 3, 8, 62, 48, 2),        # two output channels, exact tiles, batch 2
    (1, 1, 1, 1, 96, 3),         # one position
]


# fused against separate launches: the two differ where the sum of squares'
# order flips a bf16 rounding of n, which can move an output by one of its
# own bf16 ulps (2^-8 of it, 3.9e-3 of max|y| at the largest outputs)
TAIL_SEP_BAR = 1e-2


def _tail_inputs(rng, Cin, Cout):
    g = (1.0 + 0.2 * rng.standard_normal(Cin)).astype(np.float32)
    be = (0.5 * rng.standard_normal(Cin)).astype(np.float32)
    w = rnd(rng, (Cout, Cin, 3, 3, 3), 1 / math.sqrt(27 * Cin), wl.BF16)
    b = rnd(rng, (Cout,), 0.1)
    return g, be, w, b


@pytest.mark.parametrize("shape", TAIL_SHAPES)
@pytest.mark.parametrize("with_cache", [False, True])
def test_rmsnorm_silu_conv_out(torch, wv, shape, with_cache):
    """norm_out -> SiLU -> conv_out in one launch against the oracle's
    norm_silu then causal_conv3d (fp64 sums, n not rounded), and, where the
    norm kernel takes the channel count (C % 32 == 0), against the library's
    two separate launches (n through memory in bf16).  beta is far from 0, so
    a pad position normalised (silu(beta)) instead of left at zero would
    show; the cache holds the norm's input."""
    N, T, H, W, Cin, Cout = shape
    rng = np.random.default_rng(sum(shape) + 7 * with_cache)
    x = rnd(rng, (N, T, H, W, Cin), 2.0, wl.BF16)
    g, be, w, b = _tail_inputs(rng, Cin, Cout)
    cache = rnd(rng, (N, 2, H, W, Cin), 2.0, wl.BF16) if with_cache else None
    ref = oracle.causal_conv3d(oracle.norm_silu(x, g, be), w, b,
                               None if cache is None else oracle.norm_silu(cache, g, be))
    wp = wv.pack_conv3d_weights(gu.to_dev(w, wl.BF16))
    xd, gd, bed, bd = gu.to_dev(x, wl.BF16), gu.to_dev(g, wl.F32), gu.to_dev(be, wl.F32), gu.to_dev(b, wl.F32)
    cd = None if cache is None else gu.to_dev(cache, wl.BF16)
    y = wv.rmsnorm_silu_conv_out(xd, gd, bed, oracle.EPS, wp, bd, cd)
    got = gu.to_host(y)
    err = gu.rel_err(got, ref)
    extra = f"pcc={gu.pcc(got, ref):.6f}"
    sep = 0.0
    if Cin % 32 == 0:
        n = wv.rmsnorm_silu(xd, gd, bed, oracle.EPS)
        nc = None if cd is None else wv.rmsnorm_silu(cd, gd, bed, oracle.EPS)
        sep = gu.rel_err(got, gu.to_host(wv.causal_conv3d(n, wp, bd, nc)))
        extra += f" vs separate launches {sep:.3e}"
    gu.report(f"norm + conv_out {shape} cache={with_cache}", err, gu.TOL_BF16, extra)
    assert got.shape == ref.shape and err <= gu.TOL_BF16
    assert sep <= TAIL_SEP_BAR


def test_rmsnorm_silu_conv_out_decoder_sampled(torch, wv):
    """The decoder's tail at the output resolution, [1,81,720,1280,96] -> 3,
    in the launch the benchmark times: against the library's separate norm
    and conv launches over the whole output, and against the oracle on
    row bands (top, middle, bottom; full width) of the first and last
    frames, each band's oracle run on its input rows and frames (a band's
    first row and frames whose neighbourhood it does not hold are not
    compared)."""
    w_ = wl.custom("tail", wl.BF16, 1, 81, 720, 1280, 96, 3)
    xd = wl.make_x_device(w_, seed=11)
    rng = np.random.default_rng(11)
    g, be, w, b = _tail_inputs(rng, 96, 3)
    wp = wv.pack_conv3d_weights(gu.to_dev(w, wl.BF16))
    gd, bed, bd = gu.to_dev(g, wl.F32), gu.to_dev(be, wl.F32), gu.to_dev(b, wl.F32)
    y = wv.rmsnorm_silu_conv_out(xd, gd, bed, oracle.EPS, wp, bd)
    n = wv.rmsnorm_silu(xd, gd, bed, oracle.EPS)
    y2 = wv.causal_conv3d(n, wp, bd)
    del n
    torch.cuda.synchronize()
    sep = (y.float() - y2.float()).abs().max().item() / y2.float().abs().max().item()
    del y2
    errs = []
    H = 720
    for (f0, f1) in [(0, 3), (78, 81)]:
        i0 = max(f0 - 2, 0)
        for (r0, r1) in [(0, 6), (357, 363), (714, 720)]:
            a0, a1 = max(r0 - 1, 0), min(r1 + 1, H)
            xc = gu.to_host(xd[:, i0:f1, a0:a1])
            ref = oracle.causal_conv3d(oracle.norm_silu(xc, g, be), w, b)
            got = gu.to_host(y[:, f0:f1, r0:r1])
            errs.append(gu.rel_err(got, ref[:, f0 - i0:, r0 - a0:r1 - a0]))
    err = max(errs)
    gu.report("norm + conv_out [1,81,720,1280,96] -> 3 sampled", err, gu.TOL_BF16,
              f"whole output vs separate launches {sep:.3e}")
    assert err <= gu.TOL_BF16 and sep <= TAIL_SEP_BAR
    del xd, y
    torch.cuda.empty_cache()
